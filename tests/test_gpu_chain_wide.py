"""The state-chain kernel's two workgroup shapes give the same bits.

Batches with more than 32 (sequence, head) chains run the chain with two
16-column blocks of the state per workgroup; smaller ones with one.  Each
block's arithmetic is the same in both (the same fragments, products and
order), so a batch run with the two-block shape must equal, bit for bit, its
rows run one at a time with the one-block shape, and both must meet the
oracle's tolerances.
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests.parity import compare, run_gpu, run_oracle, say, to_np

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


@pytest.mark.parametrize("B,T,H,init,final", [
    (5, 64 * 6 + 23, 8, "fp32", "fp32"),   # 40 chains: two-block; each row alone: 8 chains
    (3, 64 * 4, 12, "bf16", "bf16"),       # 36 chains, whole chunks, bf16 states
])
def test_two_block_equals_one_block(B, T, H, init, final):
    w = W.make("wide", B, T, H, 7000 + B * T + H, lower_bound=-5.0, init=init, final=final)
    out, fin = run_gpu(w)
    say("case wide: B=%d T=%d H=%d (%d chains)" % (B, T, H, B * H))
    ro, rf = run_oracle(w)
    res = compare(to_np(out), ro, to_np(fin), rf, w.final_state_dtype, "wide")
    say("  vs oracle %s" % res)
    for b in range(B):
        wb = W.make("wide-row", 1, T, H, 1, lower_bound=-5.0, init=init, final=final)
        wb.q, wb.k, wb.v, wb.g, wb.beta = (x[b:b + 1].clone() for x in (w.q, w.k, w.v, w.g, w.beta))
        wb.A_log, wb.dt_bias = w.A_log, w.dt_bias
        wb.initial_state = w.initial_state[b:b + 1].clone()
        ob, fb = run_gpu(wb)
        same = torch.equal(_bits(ob), _bits(out[b:b + 1])) and torch.equal(_bits(fb), _bits(fin[b:b + 1]))
        say("  row %d alone (%d chains) equal: %s" % (b, H, same))
        assert same
