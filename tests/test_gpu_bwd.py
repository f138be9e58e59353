"""The backward pass (kda_bwd) against the oracle's fp64 gradient, element by
element, through the C ABI.

Tolerances, per gradient tensor: relative RMS (over the whole tensor) and the
largest absolute error relative to the largest reference entry.  The backward
recomputes the forward from its fp16 intermediates (so the states it
differentiates through carry the forward's ~5e-4 relative error) and runs every
product of the gradient on the fp32 matrix cores; a gradient's error is of the
order of that state error, so it is held to the forward output's relative-RMS
bar, 5e-3, and to 2e-2 of its largest entry.  Where the gate clamp decides
whether g receives a gradient, the fp64 oracle and the fp32 kernel may decide
differently for inputs within rounding of the kink: entries of dg whose
unclamped log-decay lies within 1e-4 of lower_bound are left out of the dg
comparison."""
import dataclasses
import math

import numpy as np
import pytest
import torch

import gated_delta_rule_110_amd as kda
import oracle
import workloads as W
from tests.parity import say

pytestmark = pytest.mark.gpu

GRAD_REL_RMS = 5e-3
GRAD_MAX_ABS_REL = 2e-2
NAMES = ["dq", "dk", "dv", "dg", "dbeta", "d_initial_state", "dA_log", "ddt_bias"]
REF_NAME = {"d_initial_state": "d_initial"}


def _gpu(w, d_out, d_fin, **kw):
    wd = w.to("cuda")
    res = kda.bwd(wd.q, wd.k, wd.v, wd.g, wd.beta, w.scale, wd.A_log, wd.dt_bias, w.lower_bound,
                  d_out.cuda(), d_final_state=None if d_fin is None else d_fin.cuda(),
                  initial_state=wd.initial_state, cu_seqlens=wd.cu_seqlens, **kw)
    torch.cuda.synchronize()
    return {k: (None if v is None else v.cpu().double().numpy()) for k, v in res.items()}


def _oracle(w, d_out, d_fin):
    return oracle.bwd(w.q, w.k, w.v, w.g, w.beta, w.scale, w.A_log, w.dt_bias, w.lower_bound, d_out,
                      d_final=d_fin, initial_state=w.initial_state, cu_seqlens=w.cu_seqlens)


def _near_kink(w):
    x = w.g.double().numpy() + w.dt_bias.double().numpy()[None, None]
    with np.errstate(invalid="ignore"):
        z = -np.exp(w.A_log.double().numpy())[None, None, :, None] * np.logaddexp(0.0, x)
        return np.abs(z - w.lower_bound) < 1e-4


def _compare(got, ref, w, label):
    near = _near_kink(w)
    stats = {}
    for name in NAMES:
        g_, r_ = got[name], ref[REF_NAME.get(name, name)]
        if name == "dg":
            g_, r_ = np.where(near, 0.0, g_), np.where(near, 0.0, r_)
        assert np.isfinite(g_).all(), (label, name, "non-finite")
        if r_.size == 0:
            continue
        nr = float(np.linalg.norm(r_))
        rel = float(np.linalg.norm(g_ - r_)) / nr if nr > 0 else float(np.linalg.norm(g_))
        mx = float(np.abs(g_ - r_).max()) / max(float(np.abs(r_).max()), 1e-30)
        stats[name] = (rel, mx)
    say("%s: %s" % (label, " ".join("%s %.2e/%.2e" % (k, a, b) for k, (a, b) in stats.items())))
    for name, (rel, mx) in stats.items():
        assert rel <= GRAD_REL_RMS, (label, name, rel)
        assert mx <= GRAD_MAX_ABS_REL, (label, name, mx)


CASES = {
    # ragged last chunk, three chunks, fp32 states
    "fixed": lambda: (W.make("bwd_fixed", 2, 150, 3, 7001, init="fp32", final="fp32"), 7101, "fp32"),
    # packed with an empty and a one-chunk sequence, bf16 states
    "packed": lambda: (W.make("bwd_packed", 1, 265, 2, 7002, init="bf16", final="bf16",
                              seqlens=[37, 0, 163, 65]), 7102, "bf16"),
    # no states at all
    "nostate": lambda: (W.make("bwd_nostate", 1, 64, 2, 7003, init=None, final=None), 7103, None),
    # no decay
    "lb0": lambda: (W.make("bwd_lb0", 1, 200, 2, 7004, lower_bound=0.0, init="fp32"), 7104, "fp32"),
    # weak decay, spread b
    "weak": lambda: (W.make("bwd_weak", 1, 300, 2, 7005, lower_bound=-1.0, g_mean=-2.0, beta_std=3.0,
                            init="fp32"), 7105, "fp32"),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_bwd_matches_oracle(case):
    w, seed, fin = CASES[case]()
    d_out, d_fin = W.loss_grads(w, seed, final=fin)
    say("bwd %s: B=%d T=%d H=%d N=%d" % (case, w.B, w.T, w.H, w.N))
    got = _gpu(w, d_out, d_fin)
    ref = _oracle(w, d_out, d_fin)
    _compare(got, ref, w, case)


def test_bwd_empty_batch():
    # T = 0: the initial state's gradient is the final state's, everything else is empty or zero
    w = W.make("bwd_empty", 2, 0, 2, 7006, init="fp32", final="fp32")
    d_out, d_fin = W.loss_grads(w, 7106, final="fp32")
    got = _gpu(w, d_out, d_fin)
    assert np.array_equal(got["d_initial_state"], d_fin.double().numpy())
    assert not got["dA_log"].any() and not got["ddt_bias"].any()


def test_bwd_launch_pieces_and_determinism():
    w = W.make("bwd_pieces", 1, 330, 3, 7007, init="fp32", final="fp32", seqlens=[100, 1, 229])
    d_out, d_fin = W.loss_grads(w, 7107, final="fp32")
    a = _gpu(w, d_out, d_fin)
    b = _gpu(w, d_out, d_fin)
    c = _gpu(w, d_out, d_fin, launch_piece=1)
    for name in NAMES:
        assert np.array_equal(a[name], b[name]), name
        assert np.array_equal(a[name], c[name]), name


def test_bwd_full_size_heads():
    # T = 8192, H = 32 (the headline forward shape) on the GPU; the oracle on heads 0 and 31
    w = W.config(1)
    d_out, d_fin = W.loss_grads(w, 7108, final="fp32")
    say("bwd full: %s" % w.name)
    got = _gpu(w, d_out, d_fin)
    heads = [0, w.H - 1]
    ws = w.head_slice(heads)
    idx = torch.tensor(heads)
    ref = _oracle(ws, d_out.index_select(2, idx).contiguous(), d_fin.index_select(1, idx).contiguous())
    sub = {}
    for name in NAMES:
        x = got[name]
        if name in ("dq", "dk", "dv", "dg"):
            sub[name] = x[:, :, heads]
        elif name == "dbeta":
            sub[name] = x[:, :, heads]
        elif name == "d_initial_state":
            sub[name] = x[:, heads]
        else:
            sub[name] = x[heads]
    _compare(sub, ref, ws, "full")


def _with_extremes(w, seed):
    """The same workload with the activations' extreme inputs planted (the forward's edge
    cases, here for the gradient): beta = +inf (b = 1) and -inf (b = 0) tokens, gate inputs
    g = +inf (clamped), -inf (no decay) and far beyond fp32 exp overflow, and all-zero q and
    k rows inside chunks.  Where the gate is clamped, or b is 0 or 1, no gradient reaches
    g or beta; a zero row's norm is the epsilon's."""
    rng = np.random.default_rng(seed)
    q, k, g, be = w.q.clone(), w.k.clone(), w.g.clone(), w.beta.clone()
    B, T, H, K = q.shape
    inf = float("inf")
    for tokens, val in ((rng.choice(T, 6, replace=False), inf), (rng.choice(T, 6, replace=False), -inf)):
        be[:, tokens] = val
    gi = rng.choice(T, 5, replace=False)
    g[:, gi, :, :16] = inf
    g[:, gi, :, 16:32] = -inf
    g[:, gi, :, 32:48] = 100.0
    zq, zk = rng.choice(T, 3, replace=False), rng.choice(T, 3, replace=False)
    q[:, zq] = 0
    k[:, zk] = 0
    return dataclasses.replace(w, q=q, k=k, g=g, beta=be,
                               A_log=torch.full_like(w.A_log, -8.0))  # so that g = 100 stays above lb


@pytest.mark.parametrize("lb", [-5.0, -0.5])
def test_bwd_activation_extremes(lb):
    w = _with_extremes(W.make("bwd_extremes", 2, 200, 2, 7009, lower_bound=lb, init="fp32", final="fp32"), 7209)
    d_out, d_fin = W.loss_grads(w, 7109, final="fp32")
    say("bwd extremes lb=%g" % lb)
    got = _gpu(w, d_out, d_fin)
    ref = _oracle(w, d_out, d_fin)
    _compare(got, ref, w, "extremes lb=%g" % lb)
    # b = 0 or 1: no gradient reaches beta
    be = w.beta.float().numpy()
    assert not got["dbeta"][np.isinf(be)].any()


@pytest.mark.parametrize("case", ["packed", "split"])
def test_bwd_graph_replays_match_eager(case):
    # with a caller-owned workspace and outputs the backward enqueues kernels only, so it can be
    # captured once and replayed; every replay, with the outputs and workspace clobbered eagerly
    # in between, must equal the eager call bit for bit (a packed batch; split chains)
    if case == "packed":
        w = W.make("bwd_graph", 1, 260, 3, 7010, init="fp32", final="fp32", seqlens=[100, 0, 97, 63])
        segs = 0
    else:
        w = W.make("bwd_graph_split", 2, 64 * 12 + 5, 2, 7014, init="fp32", final="fp32")
        segs = 3
    d_out, d_fin = W.loss_grads(w, 7110, final="fp32")
    wd = w.to("cuda")
    d_out, d_fin = d_out.cuda(), d_fin.cuda()
    nbytes = kda.bwd_workspace_size(w.B, w.T, w.H, num_seqs=w.N, chain_segments=segs)

    def buffers():
        outs = {n: torch.empty(sh, dtype=torch.float32, device="cuda") for n, sh in
                (("dq", (w.B, w.T, w.H, w.K)), ("dk", (w.B, w.T, w.H, w.K)), ("dv", (w.B, w.T, w.H, w.V)),
                 ("dg", (w.B, w.T, w.H, w.K)), ("dbeta", (w.B, w.T, w.H)), ("dA_log", (w.H,)),
                 ("ddt_bias", (w.H, w.K)), ("d_initial_state", (w.N, w.H, w.K, w.V)))}
        return torch.empty(nbytes, dtype=torch.uint8, device="cuda"), outs

    def call(ws, outs):
        kda.bwd(wd.q, wd.k, wd.v, wd.g, wd.beta, w.scale, wd.A_log, wd.dt_bias, w.lower_bound, d_out,
                d_final_state=d_fin, initial_state=wd.initial_state, cu_seqlens=wd.cu_seqlens, workspace=ws,
                outputs=outs, chain_segments=segs)

    ws_e, eager = buffers()
    call(ws_e, eager)
    torch.cuda.synchronize()
    ws, outs = buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(ws, outs)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(ws, outs)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs.values():
            t.fill_(float("nan"))
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in outs:
            assert torch.equal(outs[n], eager[n]), (rep, n)


def test_bwd_many_short_sequences():
    # a packed batch of 40 sequences of 1 to 150 tokens (some empty), bf16 states
    rng = np.random.default_rng(7011)
    lens = [int(x) for x in rng.integers(0, 151, 40)]
    lens[3], lens[17] = 0, 1
    w = W.make("bwd_short", 1, sum(lens), 2, 7011, init="bf16", final="bf16", seqlens=lens)
    d_out, d_fin = W.loss_grads(w, 7111, final="bf16")
    say("bwd short: N=%d T=%d" % (w.N, w.T))
    got = _gpu(w, d_out, d_fin)
    ref = _oracle(w, d_out, d_fin)
    _compare(got, ref, w, "short")


def test_bwd_long_chain():
    # 65536 tokens (1024 chunks in each reverse chain), g ~ N(-1, 1) as the 128K workload draws
    # it: the gradient state is carried through the whole chain without drifting from the oracle,
    # unsplit and in the automatic split (16 segments of 64 chunks at H = 2)
    w = W.make("bwd_long", 1, 65536, 2, 7012, init="fp32", final="fp32", g_mean=-1.0)
    d_out, d_fin = W.loss_grads(w, 7112, final="fp32")
    assert kda.chain_segments_for(w.B, w.T, w.H) == 16
    ref = _oracle(w, d_out, d_fin)
    for segs in (1, 0):
        say("bwd long: T=%d H=%d chain_segments=%d" % (w.T, w.H, segs))
        got = _gpu(w, d_out, d_fin, chain_segments=segs)
        _compare(got, ref, w, "long segs=%d" % segs)


_SPLIT_REF = {}


@pytest.mark.parametrize("segs,states", [(3, "fp32"), (4, "bf16"), (41, "fp32"), (4, None)])
def test_bwd_split_chains(segs, states):
    # split chains in the backward: the forward's segment maps, the reverse chain of every
    # segment from a zero gradient, the scan with the maps transposed, the reverse chain from
    # the gradient leaving every segment.  Two rows of 41 chunks (the last ragged) in 3, 4 and
    # 41 (one chunk each) segments; bf16 states; no states and no initial-state gradient.
    key = states
    if key not in _SPLIT_REF:
        w = W.make("bwd_split", 2, 64 * 40 + 17, 2, 7013, init=states, final=states)
        d_out, d_fin = W.loss_grads(w, 7113, final=states)
        _SPLIT_REF[key] = (w, d_out, d_fin, _oracle(w, d_out, d_fin), _gpu(w, d_out, d_fin, chain_segments=1))
    w, d_out, d_fin, ref, unsplit = _SPLIT_REF[key]
    assert kda.chain_segments_for(w.B, w.T, w.H, segs) == segs
    say("bwd split: segs=%d states=%s" % (segs, states))
    got = _gpu(w, d_out, d_fin, chain_segments=segs, with_d_initial=states is not None)
    if states is None:
        assert got["d_initial_state"] is None
        got["d_initial_state"] = unsplit["d_initial_state"]
    _compare(got, ref, w, "split segs=%d states=%s" % (segs, states))
    # the split only changes rounding: close to the unsplit gradient
    for name in NAMES:
        a, b = got[name], unsplit[name]
        scale_ = max(float(np.abs(b).max()), 1e-30)
        assert float(np.abs(a - b).max()) / scale_ <= 2e-3, (name, segs)


_FWD_WS_CASES = {
    # (workload, loss-gradient seed and final-state dtype, forward keywords, backward keywords)
    "fixed": lambda: CASES["fixed"]() + ({}, {}),
    "packed": lambda: CASES["packed"]() + ({}, {}),
    "split": lambda: (W.make("bwd_fws_split", 2, 64 * 40 + 17, 2, 7014, init="fp32", final="fp32"), 7114,
                      "fp32", {"chain_segments": 3}, {"chain_segments": 3}),
    # a forward left unsplit, a backward split in 3: the intermediates do not depend on the split
    "split_unsplit": lambda: (W.make("bwd_fws_split", 2, 64 * 40 + 17, 2, 7014, init="fp32", final="fp32"),
                              7114, "fp32", {"chain_segments": 1}, {"chain_segments": 3}),
    # the pipelined forward writes the same intermediates
    "pipelined": lambda: (W.make("bwd_fws_pipe", 1, 300, 8, 7015, init="bf16", final="fp32"), 7115, "fp32",
                          {"pipeline": 1}, {}),
}


@pytest.mark.parametrize("case", sorted(_FWD_WS_CASES))
def test_bwd_reads_forward_workspace(case):
    # kda_desc_t::forward_workspace: the backward reads the intra-chunk intermediates a forward
    # call left in its workspace instead of recomputing them, and returns the same bits
    w, seed, fin, fkw, bkw = _FWD_WS_CASES[case]()
    if "pipeline" in fkw:
        assert kda.pipelined_for(w.B, w.T, w.H, pipeline=1)
    d_out, d_fin = W.loss_grads(w, seed, final=fin)
    wd = w.to("cuda")
    ws = torch.empty(kda.workspace_size(w.B, w.T, w.H, w.N, **fkw), dtype=torch.uint8, device="cuda")
    say("bwd forward_workspace %s: B=%d T=%d H=%d N=%d" % (case, w.B, w.T, w.H, w.N))
    kda.fwd(wd.q, wd.k, wd.v, wd.g, wd.beta, w.scale, None, wd.A_log, wd.dt_bias, w.lower_bound,
            wd.initial_state, None, wd.cu_seqlens, workspace=ws, **fkw)
    ref = _gpu(w, d_out, d_fin, **bkw)
    got = _gpu(w, d_out, d_fin, forward_workspace=ws, **bkw)
    for name in NAMES:
        if ref[name] is None:
            assert got[name] is None, name
            continue
        assert np.array_equal(got[name], ref[name]), (case, name)
    # the intermediates are read, not recomputed: zeros in their place change the gradient
    zeros = torch.zeros_like(ws)
    bad = _gpu(w, d_out, d_fin, forward_workspace=zeros, **bkw)
    assert not np.array_equal(bad["dq"], ref["dq"]), case


_FWD_STATES_CASES = {
    "fixed": lambda: CASES["fixed"]() + ({}, {}),
    "packed": lambda: CASES["packed"]() + ({}, {}),
    "nostate": lambda: CASES["nostate"]() + ({}, {}),
    "split": lambda: (W.make("bwd_fws_split", 2, 64 * 40 + 17, 2, 7014, init="fp32", final="fp32"), 7114,
                      "fp32", {"chain_segments": 3}, {"chain_segments": 3}),
    # a forward that asks for the pipelined form runs the two-kernel one when it saves states
    "pipelined": lambda: (W.make("bwd_fws_pipe", 1, 300, 8, 7015, init="bf16", final="fp32"), 7115, "fp32",
                          {"pipeline": 1}, {}),
}


@pytest.mark.parametrize("case", sorted(_FWD_STATES_CASES))
def test_bwd_reads_forward_states(case):
    # kda_desc_t::save_states: the forward also stores the state entering every chunk, and the
    # backward reads the states and the intermediates from its workspace and recomputes nothing;
    # the forward's outputs and the gradients are the same bits as without
    w, seed, fin, fkw, bkw = _FWD_STATES_CASES[case]()
    d_out, d_fin = W.loss_grads(w, seed, final=fin)
    wd = w.to("cuda")
    nbytes = kda.workspace_size(w.B, w.T, w.H, w.N, save_states=True, **fkw)
    assert nbytes > kda.workspace_size(w.B, w.T, w.H, w.N, **fkw)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    say("bwd forward states %s: B=%d T=%d H=%d N=%d" % (case, w.B, w.T, w.H, w.N))
    fin_t = None if w.final_state_dtype is None else \
        torch.empty((w.N, w.H, 128, 128), dtype=w.final_state_dtype, device="cuda")
    o1, f1 = kda.fwd(wd.q, wd.k, wd.v, wd.g, wd.beta, w.scale, None, wd.A_log, wd.dt_bias, w.lower_bound,
                     wd.initial_state, fin_t, wd.cu_seqlens, workspace=ws, save_states=True, **fkw)
    o2, f2 = kda.fwd(wd.q, wd.k, wd.v, wd.g, wd.beta, w.scale, None, wd.A_log, wd.dt_bias, w.lower_bound,
                     wd.initial_state, None if fin_t is None else torch.empty_like(fin_t), wd.cu_seqlens,
                     **{k: v for k, v in fkw.items() if k != "pipeline"})
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    if f1 is not None:
        assert torch.equal(f1, f2)
    ref = _gpu(w, d_out, d_fin, **bkw)
    got = _gpu(w, d_out, d_fin, forward_workspace=ws, forward_states=True, **bkw)
    for name in NAMES:
        if ref[name] is None:
            assert got[name] is None, name
            continue
        assert np.array_equal(got[name], ref[name]), (case, name)
    # the states are read, not recomputed: zeros in the workspace change the gradient (not with
    # split chains, whose segment table the workspace holds too, nor for one chunk from a zero
    # state, where the only state read is zero either way)
    if "chain_segments" not in bkw and case != "nostate":
        bad = _gpu(w, d_out, d_fin, forward_workspace=torch.zeros_like(ws), forward_states=True, **bkw)
        assert not np.array_equal(bad["dq"], ref["dq"]), case
