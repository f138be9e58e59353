"""Value range of the GPU path.  The intra kernel hands U (built from b v), and
the chain kernel hands the state to the matrix cores, as fp16 operands, whose
range ends at 65504 and whose normal numbers start at 2^-14.  Values and
initial states far above and below unit scale must still meet the parity
tolerances, relative to their scale: v and the initial state are multiplied by
a power of two (exact in bf16 and fp32), so the outputs and the final state
scale by the same factor, and the oracle says by how much.  (2^-12 puts most
entries of U and of the state near the bottom of fp16's normal range and the
small ones among its subnormals.)"""
import dataclasses

import numpy as np
import pytest
import torch

import gated_delta_rule_110_amd as kda
import workloads as W
from tests.parity import OUT_MAX_ABS, OUT_REL_RMS, STATE_REL_FP32, run_gpu, run_oracle, say, to_np

pytestmark = pytest.mark.gpu


def _scaled(w, c):
    h0 = None if w.initial_state is None else w.initial_state * c
    return dataclasses.replace(w, v=(w.v.float() * c).to(torch.bfloat16), initial_state=h0)


def _check(out, fin, ro, rf, c, label):
    d = out - ro
    max_abs = float(np.abs(d).max())
    rel_rms = float(np.linalg.norm(d) / np.linalg.norm(ro))
    st = float(np.linalg.norm(fin - rf) / np.linalg.norm(rf))
    say("  %s x%g: out max-abs %.3e (bound %.3e) rel-rms %.3e state rel %.3e" %
        (label, c, max_abs, OUT_MAX_ABS * c, rel_rms, st))
    assert np.isfinite(out).all() and np.isfinite(fin).all(), label
    assert max_abs <= OUT_MAX_ABS * c and rel_rms <= OUT_REL_RMS and st <= STATE_REL_FP32, label


@pytest.mark.parametrize("c", [64, 512, 2.0 ** -12])
@pytest.mark.parametrize("case", ["fixed", "packed"])
def test_forward_scaled_values(case, c):
    if case == "fixed":
        w = W.make("range", 2, 300, 4, 7601, lower_bound=-5.0, init="fp32", final="fp32")
    else:
        w = W.make("range", 1, 333, 4, 7602, lower_bound=-1.0, init="fp32", final="fp32",
                   seqlens=[200, 5, 128])
    ws = _scaled(w, c)
    assert torch.equal(ws.v.float(), w.v.float() * c)  # the scaling is exact
    say("case value range %s x%g" % (case, c))
    out, fin = run_gpu(ws)
    ro, rf = run_oracle(ws)
    _check(to_np(out), to_np(fin), ro, rf, c, case)


@pytest.mark.parametrize("c", [64, 512, 2.0 ** -12])
def test_decode_scaled_values(c):
    N, H = 6, 5
    w = _scaled(W.make("range_decode", N, 1, H, 7603, lower_bound=-4.0, init="fp32", final="fp32"), c)
    say("case decode value range x%g" % c)
    wd = w.to("cuda")
    out, fin = kda.decode(wd.q, wd.k, wd.v, wd.g, wd.beta, w.scale, None, wd.A_log, wd.dt_bias,
                          w.lower_bound, wd.initial_state, torch.empty_like(wd.initial_state))
    torch.cuda.synchronize()
    ro, rf = run_oracle(w)
    _check(to_np(out), to_np(fin), ro, rf, c, "decode")
