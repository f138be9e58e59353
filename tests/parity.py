"""Helpers shared by the GPU parity tests: run the library and the oracle on
one workload and compare them with the stated tolerances."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import gated_delta_rule_110_amd as kda

# Tolerances: bf16 outputs within max-abs 2e-2 and relative RMS 5e-3 of the
# fp64 oracle; an fp32 final state within relative 1e-3 (Frobenius), over the
# whole tensor and for every (sequence, head) on its own, so that one bad short
# sequence of a packed batch is not diluted by the long ones; a bf16 final state
# within relative 5e-3 the same way, since rounding the exact state to bf16
# alone costs about 1.7e-3.
OUT_MAX_ABS = 2e-2
OUT_REL_RMS = 5e-3
STATE_REL_FP32 = 1e-3
STATE_REL_BF16 = 5e-3


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(w, device="cuda", workspace=None, out=None, final=None, chain_segments=0, launch_piece=0, pipeline=0):
    wd = w.to(device)
    if final is None and w.final_state_dtype is not None:
        final = torch.empty((w.N, w.H, w.K, w.V), dtype=w.final_state_dtype, device=device)
    out, fin = kda.fwd(wd.q, wd.k, wd.v, wd.g, wd.beta, w.scale, out, wd.A_log, wd.dt_bias,
                       w.lower_bound, wd.initial_state, final, wd.cu_seqlens, workspace=workspace,
                       chain_segments=chain_segments, launch_piece=launch_piece, pipeline=pipeline)
    torch.cuda.synchronize()
    return out, fin


def to_np(t):
    return None if t is None else t.detach().float().cpu().double().numpy()


def run_oracle(w, threads: int = 0):
    return oracle.fwd(w.q, w.k, w.v, w.g, w.beta, w.scale, w.A_log, w.dt_bias, w.lower_bound,
                      initial_state=w.initial_state, cu_seqlens=w.cu_seqlens, num_threads=threads)


def compare(out_gpu, out_ref, fin_gpu=None, fin_ref=None, fin_dtype=None, label=""):
    """Return a dict of error metrics and assert the tolerances."""
    res = {}
    d = out_gpu - out_ref
    res["out_max_abs"] = float(np.abs(d).max()) if d.size else 0.0
    nref = float(np.linalg.norm(out_ref))
    res["out_rel_rms"] = float(np.linalg.norm(d) / nref) if nref > 0 else float(np.linalg.norm(d))
    assert np.isfinite(out_gpu).all(), label + ": non-finite outputs"
    assert res["out_max_abs"] <= OUT_MAX_ABS, (label, res)
    assert res["out_rel_rms"] <= OUT_REL_RMS, (label, res)
    if fin_gpu is not None:
        tol = STATE_REL_BF16 if fin_dtype == torch.bfloat16 else STATE_REL_FP32
        nf = float(np.linalg.norm(fin_ref))
        df = float(np.linalg.norm(fin_gpu - fin_ref))
        res["state_rel"] = df / nf if nf > 0 else df
        worst = 0.0
        for n in range(fin_ref.shape[0]):
            for h in range(fin_ref.shape[1]):
                nr = np.linalg.norm(fin_ref[n, h])
                if nr > 0:
                    worst = max(worst, float(np.linalg.norm(fin_gpu[n, h] - fin_ref[n, h]) / nr))
        res["state_rel_worst"] = worst
        assert np.isfinite(fin_gpu).all(), label + ": non-finite state"
        assert res["state_rel"] <= tol, (label, res)
        assert res["state_rel_worst"] <= tol, (label, res)
    say("  %s %s" % (label, {k: "%.3e" % v for k, v in res.items()}))
    return res
