"""KDA_VALIDATE=1: kda_fwd checks the contents of cu_seqlens on the host.

Malformed tables (first entry not 0, a decreasing pair, a last entry short of
T) must be refused with KDA_ERR_SHAPE before anything is launched, so the
output and the final state keep the values they had; a well-formed table must
give the same bits as without the check.  Every malformed table here keeps its
entries within [0, T], so that even a launch would stay inside the tensors.
"""
import pytest
import torch

import gated_delta_rule_110_amd as kda
import workloads as W
from tests.parity import run_gpu, say

pytestmark = pytest.mark.gpu


def _packed():
    lens = [37, 64, 0, 129, 5]
    return W.make("validate", 1, sum(lens), 3, 7301, init="fp32", final="fp32", seqlens=lens)


def test_valid_table_same_bits(monkeypatch):
    w = _packed()
    out0, fin0 = run_gpu(w)
    monkeypatch.setenv("KDA_VALIDATE", "1")
    out1, fin1 = run_gpu(w)
    say("case validate: well-formed table, equal=%s" % (torch.equal(out0.view(torch.int16), out1.view(torch.int16))
                                                        and torch.equal(fin0, fin1)))
    assert torch.equal(out0.view(torch.int16), out1.view(torch.int16)) and torch.equal(fin0, fin1)


@pytest.mark.parametrize("bad", ["first_not_zero", "decreasing", "last_short"])
def test_malformed_table_refused(monkeypatch, bad):
    w = _packed()
    cu = w.cu_seqlens.clone()
    if bad == "first_not_zero":
        cu[0] = 3
    elif bad == "decreasing":
        cu[2] = cu[3] + 10            # [0, 37, 111, 101, ...]: the second sequence ends after the third
    else:
        cu[-1] = cu[-1] - 2
    assert int(cu.min()) >= 0 and int(cu.max()) <= w.T
    w.cu_seqlens = cu
    monkeypatch.setenv("KDA_VALIDATE", "1")
    wd = w.to("cuda")
    out = torch.full((w.B, w.T, w.H, w.V), 7.0, dtype=torch.bfloat16, device="cuda")
    fin = torch.full((w.N, w.H, w.K, w.V), 5.0, dtype=torch.float32, device="cuda")
    say("case validate: %s %s" % (bad, cu.tolist()))
    with pytest.raises(kda.KdaError) as ei:
        kda.fwd(wd.q, wd.k, wd.v, wd.g, wd.beta, w.scale, out, wd.A_log, wd.dt_bias, w.lower_bound,
                wd.initial_state, fin, wd.cu_seqlens)
    torch.cuda.synchronize()
    assert ei.value.status == 2
    assert bool((out.float() == 7.0).all()) and bool((fin == 5.0).all())
