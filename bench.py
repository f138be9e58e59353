"""Throughput of the KDA chunked forward pass on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2] [--no-cpu-baseline] [--bwd [--keep-intermediates]]

One step = one kda_fwd call (chunk table when packed, intra-chunk kernel,
state-chain kernel) over the whole workload, with inputs already resident in
HBM.  W untimed steps, then K timed steps between device synchronisations.
Prints one JSON line.  Per-kernel device time comes from HIP events that
kda_fwd records on its stream around each kernel, on one timed step in ten
(the records cost about 15 us per step, so the other steps run without them).

The default workload is the long single-sequence prefill: B=1, T=8192, H=32,
K=V=128, bf16 inputs drawn N(0,1), lower_bound=-5, no initial state, bf16
final state.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import torch  # noqa: E402

import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16/fp16 MFMA, vendor figure
# Algorithmic work per token-head (C = 64, K = V = 128):
#   FLOPs 6KV + C(3K + 2V) = 139,264; bytes: q, k, v, g in (4 x 256) + beta (2) + out (256) = 1282,
#   plus the optional states (K V x 2 or 4 bytes per (sequence, head) each).
F_ALG = 6 * 128 * 128 + 64 * (3 * 128 + 2 * 128)
BYTES_ALG = 4 * 256 + 2 + 256
# The part of those bytes each kernel moves: the intra-chunk kernel reads the
# inputs, the state chain writes the outputs and reads / writes the states.
ALG_SHARE_BYTES = {"kda_intra_kernel": 4 * 256 + 2, "chain": 256}
# Interface bytes per token-head of each kernel, reading its inputs and writing
# its outputs once, the library's own intermediates included.  These are W, Qg,
# Kbar^T, U (64 x 128 fp16 each), the 6 of 8 A_qk fragments that are not
# identically zero (rows 0..31 have no entries in columns 32..63) and exp(G_n)
# (128 fp32): 70.5 KiB per 64-token chunk and head = 1128 B per token-head.
# They are reported beside the algorithmic figures (frac_interface), never as them.
INTER_BYTES = (4 * 64 * 128 * 2 + 6 * 1024 + 128 * 4) / 64.0
KERNEL_BYTES = {
    "kda_intra_kernel": 4 * 256 + 2 + INTER_BYTES,
    "kda_chain_kernel": INTER_BYTES + 256,
    "kda_chain_x2_kernel": INTER_BYTES + 256,
    # split chains (the map pass, the scan over segments and the chain with outputs, timed
    # together): the intermediates are read twice, once per chain pass
    "split_chain": 2 * INTER_BYTES + 256,
}
# Split chains also move, per (batch row, segment, head), the two fp32 maps (written by the
# map pass, read by the scan) and the entering state (written by the scan, read by the chain).
SPLIT_BYTES_PER_SEGMENT_HEAD = 2 * (2 * 128 * 128 * 4) + 2 * (128 * 128 * 4)
# The matrix-core operand types the kernels use (the I/O type is "dtype").
MFMA_OPERANDS = ("fp16 (state path and output path), bf16 hi+lo splits on the diagonal Gram blocks, "
                 "split-fp16 off-diagonal inverse blocks; fp32 accumulation")


def state_bytes(w) -> int:
    per = w.N * w.H * w.K * w.V
    b = 0
    if w.initial_state is not None:
        b += per * w.initial_state.element_size()
    if w.final_state_dtype is not None:
        b += per * (2 if w.final_state_dtype == torch.bfloat16 else 4)
    return b


def cpu_baseline(w, target_s: float = 10.0):
    """Time the fp64 oracle (the plain token recurrence, as it stands) on the host cores.

    The sample is the first T_s tokens of every sequence and all heads, run
    repeatedly until about ``target_s`` seconds of wall time have passed."""
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1)
    units = w.N * w.H
    cores = min(threads, units)

    def run(T_s):
        t0 = time.perf_counter()
        if w.cu_seqlens is not None:  # packed batch: always the whole batch
            oracle.fwd(w.q, w.k, w.v, w.g, w.beta, w.scale, w.A_log, w.dt_bias, w.lower_bound,
                       initial_state=w.initial_state, cu_seqlens=w.cu_seqlens, num_threads=threads)
        else:
            q, k, v, g, b = (t[:, :T_s].contiguous() for t in (w.q, w.k, w.v, w.g, w.beta))
            oracle.fwd(q, k, v, g, b, w.scale, w.A_log, w.dt_bias, w.lower_bound,
                       initial_state=w.initial_state, num_threads=threads)
        return time.perf_counter() - t0

    T_s = 64 if w.cu_seqlens is None else w.T
    dt = run(T_s)
    while dt < 1.0 and T_s < w.T:
        T_s = min(w.T, T_s * 4)
        dt = run(T_s)
    reps, total = 1, dt
    while total < target_s:
        total += run(T_s)
        reps += 1
    tokens = w.B * T_s * reps
    return {"value": round(tokens / total, 1), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "first %d of %d tokens of every sequence, all %d heads, fp64 token recurrence, "
                      "%d repetitions, %d OpenMP threads, %.1f s" % (T_s, w.T, w.H, reps, threads, total)}


# The files each kernel's code and launch depend on: its own source (which
# holds its launcher and grid), the shared header, the public header and the
# build flags; for split chains also kda_api.hip, which chooses the segments.
_COMMON_SOURCES = ["kda_common.h", "../_build.py"]
KERNEL_SOURCES = {
    "kda_intra_kernel": ["kda_intra.hip", "kda_intra_body.h"],
    "kda_chain_kernel": ["kda_chain.hip"],
    "kda_chain_x2_kernel": ["kda_chain.hip"],
    "kda_chunk_table_kernel": ["kda_chain.hip"],
    "split_chain": ["kda_chain.hip", "kda_segment.hip", "kda_api.hip", "kda_bwd_args.h", "../../include/kda.h"],
    "kda_decode_kernel": ["kda_decode.hip"],
    "kda_decode_stream_kernel": ["kda_decode.hip"],
    "kda_decode_split2_kernel": ["kda_decode.hip"],
    "kda_decode_split4_kernel": ["kda_decode.hip"],
    "kda_chain_save_kernel": ["kda_chain.hip"],
    "kda_bwd_prep_kernel": ["kda_bwd.hip", "kda_bwd_args.h"],
    "kda_bwd_chain_kernel": ["kda_bwd.hip", "kda_bwd_args.h"],
    "kda_bwd_main_kernel": ["kda_bwd.hip", "kda_bwd_args.h"],
    "kda_bwd_params_kernel": ["kda_bwd.hip", "kda_bwd_args.h"],
}
# The library's choice of decode kernel, mirrored to name it: states of this
# many bytes or more are streamed past the Infinity Cache; otherwise each head
# is spread over 4 column slices while that makes at most 512 workgroups, over
# 2 slices up to 1024, else one workgroup per (sequence, head).
DECODE_STREAM_STATE_BYTES = 256 << 20
DECODE_SPLIT_WORKGROUPS = 512


def decode_kernel_name(N: int, H: int) -> str:
    units = N * H
    if units * 128 * 128 * 4 >= DECODE_STREAM_STATE_BYTES:
        return "kda_decode_stream_kernel"
    if units * 4 <= DECODE_SPLIT_WORKGROUPS:
        return "kda_decode_split4_kernel"
    if units * 2 <= 2 * DECODE_SPLIT_WORKGROUPS:
        return "kda_decode_split2_kernel"
    return "kda_decode_kernel"


def copy_bandwidth(dev, mib: int = 1024, reps: int = 5) -> float:
    """Achievable HBM bandwidth: bytes read plus written per second of a plain
    streaming copy of ``mib`` MiB (the median of ``reps``), a second
    denominator beside the vendor peak.  The copy is torch's elementwise
    kernel (dst = src * 1 in fp32), which streams faster than the runtime's
    blit behind ``copy_`` (about 6.1 against 5.1 TB/s)."""
    n = mib << 20
    src = torch.ones(n // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.mul(src, 1.0, out=dst)
    times = []
    for _ in range(reps):
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        torch.mul(src, 1.0, out=dst)
        t1.record()
        torch.cuda.synchronize(dev)
        times.append(t0.elapsed_time(t1))
    ms = sorted(times)[len(times) // 2]
    del src, dst
    return 2 * n / (ms / 1e3) / 1e9


def _code_only(name: str, text: str) -> str:
    """The code of a source file without its comments and with runs of white
    space collapsed, so that editing a comment does not change a digest."""
    import re
    if name.endswith(".py"):
        text = re.sub(r"(?m)^\s*#.*$", "", text)
    else:
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
    return " ".join(text.split())


def source_digest(kernel=None) -> str:
    """sha256 over the code (comments aside) of the HIP sources, headers and
    build flags the library is built from: all of them, or those ``kernel`` is
    built and launched from."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_delta_rule_110_amd", "csrc")
    names = (sorted(os.listdir(csrc)) + ["../../include/kda.h", "../_build.py"] if kernel is None
             else sorted(KERNEL_SOURCES[kernel]) + _COMMON_SOURCES)
    for name in names:
        path = os.path.normpath(os.path.join(csrc, name))
        if os.path.isfile(path):
            h.update(name.encode())
            with open(path, encoding="utf-8") as f:
                h.update(_code_only(name, f.read()).encode())
    return h.hexdigest()


def traffic_path(workload_name: str) -> str:
    return os.path.join(ROOT, "profiles", "traffic_%s.json" % workload_name)


def write_traffic(pmc_dir: str, workload_name: str) -> dict:
    """Summarise rocprofv3 --pmc runs into profiles/traffic_<workload>.json.

    pmc_dir holds four rocprofv3 CSV output folders: fetch/ (FETCH_SIZE on
    bench.py), write/ (WRITE_SIZE on bench.py), calf/ and calw/ (the same
    counters on ``bench.py --copy-calibration MIB``).  Both counters are in KiB
    per dispatch; each is scaled by (copy bytes) / (counter bytes of the copy
    kernel), so that a plain copy of known size reads as its true size."""
    import csv
    import glob

    def per_kernel(sub):
        sums, counts = {}, {}
        for f in glob.glob(os.path.join(pmc_dir, sub, "*counter_collection.csv")):
            for r in csv.DictReader(open(f)):
                name = r["Kernel_Name"]
                key = None
                for kn in ("kda_intra_kernel", "kda_chain_kernel", "kda_chain_x2_kernel", "kda_chunk_table_kernel",
                           "kda_decode_kernel", "kda_decode_stream_kernel", "kda_decode_split2_kernel",
                           "kda_decode_split4_kernel", "kda_chain_save_kernel", "kda_bwd_prep_kernel",
                           "kda_bwd_chain_kernel", "kda_bwd_main_kernel", "kda_bwd_params_kernel", "copyBuffer"):
                    if kn in name:
                        key = kn
                if key is None:
                    continue
                sums[key] = sums.get(key, 0.0) + float(r["Counter_Value"])
                counts[key] = counts.get(key, 0) + 1
        return {k: sums[k] / counts[k] for k in sums}

    with open(os.path.join(pmc_dir, "calibration_bytes.txt")) as f:
        cal_bytes = float(f.read().strip())
    cf, cw = per_kernel("calf"), per_kernel("calw")
    scale_f = cal_bytes / (cf["copyBuffer"] * 1024.0)
    scale_w = cal_bytes / (cw["copyBuffer"] * 1024.0)
    fe, wr = per_kernel("fetch"), per_kernel("write")
    res = {"workload": workload_name, "source_sha256": source_digest(),
           "fetch_scale": round(scale_f, 4), "write_scale": round(scale_w, 4), "kernels": {}}
    for k in fe:
        if k == "copyBuffer":
            continue
        rb = fe[k] * 1024.0 * scale_f
        wb = wr.get(k, 0.0) * 1024.0 * scale_w
        res["kernels"][k] = {"read_bytes": round(rb), "write_bytes": round(wb), "bytes": round(rb + wb)}
        if k in KERNEL_SOURCES:
            res["kernels"][k]["source_sha256"] = source_digest(k)
    with open(traffic_path(workload_name), "w") as f:
        json.dump(res, f, indent=1)
    return res


def load_traffic(workload_name: str, kernel: str):
    """HBM bytes per launch of ``kernel`` from the committed counter summary, or
    None when there is none or the kernel's sources changed since it was taken."""
    path = traffic_path(workload_name)
    if not os.path.exists(path) or kernel not in KERNEL_SOURCES:
        return None
    with open(path) as f:
        tr = json.load(f)
    k = tr.get("kernels", {}).get(kernel)
    if k is None or k.get("source_sha256") != source_digest(kernel):
        return None
    return k["bytes"]


def load_limiter(kernel: str):
    """What the committed counters say bounds ``kernel`` (profiles/limiters.json),
    or None when there is no entry or the kernel's sources changed since."""
    path = os.path.join(ROOT, "profiles", "limiters.json")
    if not os.path.exists(path) or kernel not in KERNEL_SOURCES:
        return None
    with open(path) as f:
        lim = json.load(f).get(kernel)
    if lim is None or lim.get("source_sha256") != source_digest(kernel):
        return None
    return lim.get("limiter")


# The backward (kda_bwd): the forward recomputed (F_ALG), then per token-head
#   reverse state chain: scale A_qk^T dO (C V, triangular), Kbar dS, W^T dUt, Qg^T dO (2 K V each)
#   per-chunk gradient: gamma Khat S, dO S^T, Z S^T, Ut dS'^T (2 K V each); T X, T^T dUt,
#     dO Ut^T, Z Ut^T (C V each, triangular); the four Gram gradients (C K each, triangular)
#   preparation: the decayed key Gram (C K, triangular)
F_BWD_CHAIN = 64 * 128 + 3 * 2 * 128 * 128
F_BWD_MAIN = 4 * 2 * 128 * 128 + 4 * 64 * 128 + 4 * 64 * 128
F_BWD_PREP = 64 * 128
F_BWD = F_ALG + F_BWD_CHAIN + F_BWD_MAIN + F_BWD_PREP
# Algorithmic bytes per token-head: q, k, v, g, beta and d_out read (bf16), dq, dk, dv, dg (fp32)
# and dbeta (fp32) written; plus the states (initial state and d_final read, d_initial written).
BYTES_BWD = 4 * 256 + 2 + 256 + 4 * 512 + 4
MFMA_FP32_PEAK_TFLOPS = 157.3   # MI355X dense fp32 MFMA, vendor figure


def bench_bwd(kda, args, dev, wname) -> int:
    """The backward: K timed kda_bwd calls on the workload, with d_out ~ N(0, 1)
    and an fp32 d_final when the workload has a final state."""
    w_host = W.by_name(wname)
    w = w_host.to(dev)
    d_out, d_fin = W.loss_grads(w_host, 8000, final="fp32" if w.final_state_dtype is not None else None)
    d_out = d_out.to(dev)
    d_fin = None if d_fin is None else d_fin.to(dev)
    segs_req = args.chain_segments if w.cu_seqlens is None else 0
    nbytes = kda.bwd_workspace_size(w.B, w.T, w.H, num_seqs=w.N, chain_segments=segs_req)
    segs = kda.chain_segments_for(w.B, w.T, w.H, segs_req) if w.cu_seqlens is None else 1
    workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    for e in ev:
        e.record(stream)
    torch.cuda.synchronize(dev)
    ev_arr = (ctypes.c_void_p * 6)(*[ctypes.c_void_p(e.cuda_event) for e in ev])
    fws = None
    fwd_keep_ms = None
    if args.keep_intermediates:
        # a training step's backward: the forward kept its workspace, with the state entering
        # every chunk, and the backward recomputes nothing; that forward is timed here too
        fws = torch.empty(kda.workspace_size(w.B, w.T, w.H, w.N, chain_segments=segs_req, save_states=True),
                          dtype=torch.uint8, device=dev)
        fin_t = None if w.final_state_dtype is None else \
            torch.empty((w.N, w.H, 128, 128), dtype=w.final_state_dtype, device=dev)
        out_t = torch.empty(w.v.shape, dtype=torch.bfloat16, device=dev)

        def fwd_keep():
            kda.fwd(w.q, w.k, w.v, w.g, w.beta, w.scale, out_t, w.A_log, w.dt_bias, w.lower_bound,
                    w.initial_state, fin_t, w.cu_seqlens, workspace=fws, chain_segments=segs_req,
                    save_states=True)

        for _ in range(max(args.warmup, 1)):
            fwd_keep()
        torch.cuda.synchronize(dev)
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        f0.record(stream)
        for _ in range(args.steps):
            fwd_keep()
        f1.record(stream)
        torch.cuda.synchronize(dev)
        fwd_keep_ms = f0.elapsed_time(f1) / args.steps

    def step(events=None):
        return kda.bwd(w.q, w.k, w.v, w.g, w.beta, w.scale, w.A_log, w.dt_bias, w.lower_bound, d_out,
                       d_final_state=d_fin, initial_state=w.initial_state, cu_seqlens=w.cu_seqlens,
                       workspace=workspace, phase_events=events, chain_segments=segs_req,
                       forward_workspace=fws, forward_states=fws is not None)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        step(ctypes.cast(ev_arr, ctypes.c_void_p) if i == args.steps - 1 else None)
    t1.record(stream)
    torch.cuda.synchronize(dev)
    ms = t0.elapsed_time(t1) / args.steps
    # with split chains the two chain entries time the three launches of each side
    names = ["fwd_intra", "fwd_chain_save", "kda_bwd_prep_kernel", "kda_bwd_chain_kernel", "kda_bwd_main_kernel"]
    kernel_ms = {n: round(ev[i].elapsed_time(ev[i + 1]), 5) for i, n in enumerate(names)}
    tok_heads = w.B * w.T * w.H
    flops = {"kda_bwd_prep_kernel": F_BWD_PREP, "kda_bwd_chain_kernel": F_BWD_CHAIN,
             "kda_bwd_main_kernel": F_BWD_MAIN}
    per_kernel = {n: {"alg_tflops": round(f * tok_heads / (kernel_ms[n] / 1e3) / 1e12, 2),
                      "frac_fp32_mfma": round(f * tok_heads / (kernel_ms[n] / 1e3) / 1e12 / MFMA_FP32_PEAK_TFLOPS, 4),
                      "traffic": load_traffic("bwd_" + wname, n)}
                  for n, f in flops.items()}
    dom = max(flops, key=lambda n: kernel_ms[n])
    achieved = flops[dom] * tok_heads / (kernel_ms[dom] / 1e3) / 1e12
    sb = state_bytes(w) + (0 if d_fin is None else w.N * w.H * 128 * 128 * 4) + w.N * w.H * 128 * 128 * 4
    alg_bytes = BYTES_BWD * tok_heads + sb
    result = {
        "metric": ("KDA backward tokens/s (gradient of the prefill, from the forward's kept intermediates "
                   "and states)"
                   if fws is not None else
                   "KDA backward tokens/s (gradient of the prefill, recomputing the forward)"),
        "value": round(w.B * w.T / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 in, fp32 gradients", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "H": w.H, "K": w.K, "V": w.V, "num_seqs": w.N,
                   "chain_segments": segs, "forward_intermediates": "kept" if fws is not None else "recomputed"},
        "kernel_ms": kernel_ms,
        # with kept intermediates: the forward that keeps them, and forward + backward
        "forward_keep_ms": None if fwd_keep_ms is None else round(fwd_keep_ms, 5),
        "train_step_ms": None if fwd_keep_ms is None else round(fwd_keep_ms + ms, 5),
        "tflops_alg": round(F_BWD * tok_heads / (ms / 1e3) / 1e12, 2),
        "gbs_alg": round(alg_bytes / (ms / 1e3) / 1e9, 1),
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_FP32_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_FP32_PEAK_TFLOPS, 4),
                     "alg_flops": flops[dom] * tok_heads, "traffic": load_traffic("bwd_" + wname, dom),
                     "limiter": load_limiter(dom), "kernels": per_kernel},
        "mfma_operands": ("per-chunk gradient: bf16 hi + lo splits of the fp32 operands (16x16x32) against S, dS', "
                          "Ut, T, dUt, fp32 (16x16x4) for the Gram gradients; preparation fp32; reverse chain fp16; "
                          "the recomputed forward as kda_fwd"),
    }
    print(json.dumps(result), flush=True)
    return 0


def decode_name(N: int, H: int) -> str:
    return "decode_N%d_H%d" % (N, H)


def bench_decode(kda, args, dev, H) -> int:
    """Decode step: N sequences x H heads, one token each, fp32 state in place,
    timed as K steps replayed from a HIP graph (eager launches reported beside).
    Algorithmic HBM bytes per step: the state read and written (2 x 64 KiB per
    head) plus q, k, v, g (4 x 256 B), beta (2 B) and out (256 B) per head."""
    N = args.decode
    w = W.make(decode_name(N, H), N, 1, H, 6000 + N, lower_bound=-5.0, init="fp32", final="fp32").to(dev)
    st = w.initial_state.clone()
    out = torch.empty((N, 1, H, 128), dtype=torch.bfloat16, device=dev)

    def step():
        kda.decode(w.q, w.k, w.v, w.g, w.beta, w.scale, out, w.A_log, w.dt_bias, w.lower_bound, st, st)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize(dev)
    eager_ms = t0.elapsed_time(t1) / args.steps
    # The same K steps captured once in a HIP graph and replayed: a serving
    # loop issues decode steps that way, and the step time is then the
    # device's rather than the host's (one Python call and launch per step).
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(args.steps):
            step()
    graph.replay()
    torch.cuda.synchronize(dev)
    t0.record()
    graph.replay()
    t1.record()
    torch.cuda.synchronize(dev)
    ms = t0.elapsed_time(t1) / args.steps
    nbytes = N * H * (2 * 128 * 128 * 4 + 4 * 256 + 2 + 256)
    gbs = nbytes / (ms / 1e3) / 1e9
    kernel = decode_kernel_name(N, H)
    print(json.dumps({"metric": "KDA decode tokens/s (one token per sequence, fp32 state in place)",
                      "value": round(N / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
                      "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
                      "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
                      "config": {"workload": "decode", "N": N, "H": H, "K": 128, "V": 128,
                                 "launch": "hip_graph of the timed steps"},
                      "eager_us_per_step": round(eager_ms * 1e3, 2),
                      "roofline": {"kernel": kernel, "bound": "hbm", "achieved": round(gbs, 1),
                                   "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                                   "traffic": load_traffic(decode_name(N, H), kernel)}}), flush=True)
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=int(os.environ.get("WORLD_SIZE", "1")))
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="2",
                    help="workload index 0..4 (default 2: T=8192, H=32) or a name from workloads.PAGES_NAMES "
                         "(the pages' H=96 / H=64 shapes) or workloads.SPLIT_NAMES (one long sequence, few heads)")
    ap.add_argument("--chain-segments", type=int, default=0, metavar="N",
                    help="split each state chain into N segments (0: the library's automatic choice, "
                         "1: never; batches without cu_seqlens)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode", type=int, default=0, metavar="N",
                    help="time the single-token recurrent step (kda_decode) for N sequences of the "
                         "chosen workload's head count, fp32 state updated in place, and exit")
    ap.add_argument("--bwd", action="store_true",
                    help="time the backward pass (kda_bwd) on the chosen workload and exit")
    ap.add_argument("--keep-intermediates", action="store_true",
                    help="with --bwd: the backward reads the intermediates and states of a forward call's "
                         "kept workspace (that forward is timed too)")
    ap.add_argument("--traffic-from", default=None, metavar="DIR",
                    help="write profiles/traffic_<workload>.json from rocprofv3 --pmc CSV folders in DIR and exit")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB five times (the "
                         "reference kernel that scales FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print("bench.py measures one GPU only: the KDA forward shards by heads or sequences with "
              "no communication, so no multi-GPU run is made (asked for %d GPUs)" % args.gpus,
              file=sys.stderr)
        return 2

    wname = W.CONFIG_NAMES[int(args.workload)] if args.workload.isdigit() else args.workload
    decode_H = W.by_name(wname).H if args.decode else 0
    if args.decode:
        wname = decode_name(args.decode, decode_H)
    if args.traffic_from:
        print(json.dumps(write_traffic(args.traffic_from, "bwd_" + wname if args.bwd else wname)))
        return 0
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}), flush=True)
        return 0

    import gated_delta_rule_110_amd as kda
    if not os.path.exists(kda.LIB_PATH):
        kda.build()

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.decode:
        return bench_decode(kda, args, dev, decode_H)
    if args.bwd:
        return bench_bwd(kda, args, dev, wname)
    w_host = W.by_name(wname)
    w = w_host.to(dev)
    out = torch.empty((w.B, w.T, w.H, w.V), dtype=torch.bfloat16, device=dev)
    final = None
    if w.final_state_dtype is not None:
        final = torch.empty((w.N, w.H, w.K, w.V), dtype=w.final_state_dtype, device=dev)
    packed = w.cu_seqlens is not None
    segs = 1 if packed else kda.chain_segments_for(w.B, w.T, w.H, args.chain_segments)
    nbytes = kda.workspace_size(w.B, w.T, w.H, num_seqs=w.N, chain_segments=args.chain_segments)
    workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)

    # Phase events: 4 per sampled step (created by a first record).  Recording
    # them costs about 15 us per step, so only one timed step in ten is
    # sampled (at least the last one); the others run uninstrumented.
    stream = torch.cuda.current_stream(dev)
    sampled = [i for i in range(args.steps) if i % 10 == 9] or [args.steps - 1]
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in sampled]
    for row in evs:
        for e in row:
            e.record(stream)
    torch.cuda.synchronize(dev)
    ev_arrays = []
    for row in evs:
        arr = (ctypes.c_void_p * 4)(*[ctypes.c_void_p(e.cuda_event) for e in row])
        ev_arrays.append(arr)

    def step(ev=None):
        kda.fwd(w.q, w.k, w.v, w.g, w.beta, w.scale, out, w.A_log, w.dt_bias, w.lower_bound,
                w.initial_state, final, w.cu_seqlens, workspace=workspace,
                phase_events=None if ev is None else ctypes.cast(ev, ctypes.c_void_p),
                chain_segments=args.chain_segments)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    wall0 = time.perf_counter()
    ev_of = dict(zip(sampled, ev_arrays))
    for i in range(args.steps):
        step(ev_of.get(i))
    t_end.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    ms = total_ms / args.steps

    intra_ms = sum(r[1].elapsed_time(r[2]) for r in evs) / len(evs)
    chain_ms = sum(r[2].elapsed_time(r[3]) for r in evs) / len(evs)
    table_ms = sum(r[0].elapsed_time(r[1]) for r in evs) / len(evs)
    tok_heads = w.B * w.T * w.H
    tokens = w.B * w.T
    tokens_per_s = tokens / (ms / 1e3)
    tflops = F_ALG * tok_heads / (ms / 1e3) / 1e12
    path_bytes = BYTES_ALG * tok_heads + state_bytes(w)
    gbs = path_bytes / (ms / 1e3) / 1e9

    # the library runs the chain with two 16-column blocks per workgroup
    # (kda_chain_x2_kernel) when one block per workgroup would need more than
    # 256 workgroups (8 per sequence and head)
    if segs > 1:
        chain_key = "split_chain"
    elif w.N * w.H * 8 > 256:
        chain_key = "kda_chain_x2_kernel"
    else:
        chain_key = "kda_chain_kernel"
    kernels = {"kda_intra_kernel": intra_ms, chain_key: chain_ms}
    def kernel_bytes(name):
        b = KERNEL_BYTES[name] * tok_heads
        if name != "kda_intra_kernel":
            b += state_bytes(w)
        if name == "split_chain":
            b += SPLIT_BYTES_PER_SEGMENT_HEAD * w.B * segs * w.H
        return b

    dom = max(kernels, key=kernels.get)
    # The roofline of the path: the algorithmic bytes of the whole forward
    # (1282 B per token-head plus the states), credited to the dominant kernel's
    # time, against the HBM peak.  Each kernel's own share of those bytes (the
    # inputs it reads, the outputs and states it writes) gives its share rate;
    # the interface rate (its reads and writes including the intermediates) is
    # reported beside them.
    alg_bytes = path_bytes

    def share_bytes(name):
        if name == "kda_intra_kernel":
            return ALG_SHARE_BYTES[name] * tok_heads
        return ALG_SHARE_BYTES["chain"] * tok_heads + state_bytes(w)

    achieved = alg_bytes / (kernels[dom] / 1e3) / 1e9
    # Which roofline bounds the path: the larger of its two floor times, the
    # algorithmic bytes at the HBM peak and the algorithmic FLOPs at the dense
    # fp16 / bf16 MFMA peak (the path's products are fp16 / bf16 MFMAs).
    floor_hbm_us = alg_bytes / (HBM_PEAK_GBS * 1e9) * 1e6
    floor_mfma_us = F_ALG * tok_heads / (MFMA_BF16_PEAK_TFLOPS * 1e12) * 1e6
    bound = "hbm" if floor_hbm_us >= floor_mfma_us else "mfma"
    copy_gbs = copy_bandwidth(dev)
    per_kernel = {}
    counter_total = 0
    for name, t in kernels.items():
        sh = share_bytes(name) / (t / 1e3) / 1e9
        gi = kernel_bytes(name) / (t / 1e3) / 1e9
        tr = load_traffic(wname, name)
        counter_total = None if (tr is None or counter_total is None) else counter_total + tr
        per_kernel[name] = {"alg_share_bytes": share_bytes(name), "share_achieved": round(sh, 1),
                            "share_frac": round(sh / HBM_PEAK_GBS, 4),
                            "interface_bytes": round(kernel_bytes(name)), "interface_achieved": round(gi, 1),
                            "frac_interface": round(gi / HBM_PEAK_GBS, 4), "traffic": tr,
                            "traffic_ratio": None if tr is None else round(tr / share_bytes(name), 3),
                            "limiter": load_limiter(name)}
    traffic = load_traffic(wname, dom)
    dom_iface = kernel_bytes(dom) / (kernels[dom] / 1e3) / 1e9

    result = {
        "metric": "KDA prefill tokens/s and MFMA TFLOP/s (% bf16 peak) at T=8K,H=32,K=V=128",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "H": w.H, "K": w.K, "V": w.V,
                   "num_seqs": w.N, "lower_bound": w.lower_bound,
                   "initial_state": None if w.initial_state is None else str(w.initial_state.dtype),
                   "final_state": None if w.final_state_dtype is None else str(w.final_state_dtype),
                   "chain_segments": segs},
        "tflops_alg": round(tflops, 2),
        "mfma_frac_alg": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "gbs_alg": round(gbs, 1),
        "hbm_frac_alg": round(gbs / HBM_PEAK_GBS, 4),
        "kernel_ms": dict(([("kda_chunk_table_kernel", round(table_ms, 5))] if packed else [])
                          + [("kda_intra_kernel", round(intra_ms, 5)), (chain_key, round(chain_ms, 5))]),
        "kernel_ms_samples": len(evs),
        "roofline": {"kernel": dom, "bound": bound,
                     **({"achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4)} if bound == "hbm" else
                        {"achieved": round(F_ALG * tok_heads / (kernels[dom] / 1e3) / 1e12, 2),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(F_ALG * tok_heads / (kernels[dom] / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}),
                     "floor_us": {"hbm": round(floor_hbm_us, 1), "mfma": round(floor_mfma_us, 1)},
                     "alg_bytes": alg_bytes, "traffic": traffic,
                     "traffic_ratio": None if counter_total is None else round(counter_total / alg_bytes, 3),
                     "frac_interface": round(dom_iface / HBM_PEAK_GBS, 4),
                     "limiter": load_limiter(dom),
                     "copy_gbs": round(copy_gbs, 1), "frac_of_copy": round(achieved / copy_gbs, 4),
                     "kernels": per_kernel},
        "mfma_operands": MFMA_OPERANDS,
        "wall_s": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w_host)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
