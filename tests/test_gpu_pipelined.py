"""The pipelined forward (kda_desc_t::pipeline = 1: intra-chunk producers and
state-chain consumers in one grid, the intermediates passed through each XCD's
L2) against the two-kernel forward and the oracle.

Both paths compute the same fp16 intermediates and run the same matrix-core
products in the same order, so their outputs and final states must be equal
bit for bit; both must meet the oracle's tolerances.  Shapes cover one and
several chains per consumer workgroup (rounds), ragged last chunks, every
state dtype, and head counts 8 to 64."""
import pytest
import torch

import gated_delta_rule_110_amd as kda
import workloads as W
from tests.parity import compare, run_gpu, run_oracle, say, to_np

pytestmark = pytest.mark.gpu

CASES = [
    # (B, T, H, init, final, lower_bound)
    (1, 64, 8, None, "fp32", -5.0),        # one chunk, one chain per XCD
    (1, 1000, 8, "fp32", "fp32", -5.0),    # ragged last chunk
    (2, 333, 16, "bf16", "bf16", -3.0),    # two chains per XCD, bf16 states
    (3, 200, 32, "fp32", None, -5.0),      # 12 chains per XCD: three rounds of four consumers
    (1, 2048, 32, None, "bf16", -5.0),
    (2, 700, 64, "fp32", "fp32", -1.0),    # 16 chains per XCD
]


@pytest.mark.parametrize("B,T,H,init,final,lb", CASES)
def test_pipelined_equals_two_kernel(B, T, H, init, final, lb):
    w = W.make("pipe", B, T, H, 9400 + T + H, lower_bound=lb, init=init, final=final)
    assert kda.pipelined_for(B, T, H, pipeline=1) and not kda.pipelined_for(B, T, H)
    say("case pipelined B=%d T=%d H=%d init=%s final=%s" % (B, T, H, init, final))
    o1, f1 = run_gpu(w, pipeline=1)
    o2, f2 = run_gpu(w)
    assert torch.equal(o1, o2), "outputs differ from the two-kernel forward"
    assert (f1 is None and f2 is None) or torch.equal(f1, f2), "final states differ"
    ro, rf = run_oracle(w)
    compare(to_np(o1), ro, to_np(f1), rf, w.final_state_dtype, "pipelined B=%d T=%d H=%d" % (B, T, H))


def test_pipelined_applies_only_where_stated():
    assert kda.pipelined_for(1, 8192, 32, pipeline=1)
    assert not kda.pipelined_for(1, 8192, 32)            # opt-in
    assert not kda.pipelined_for(1, 8192, 4, pipeline=1)  # H not a multiple of 8
    assert not kda.pipelined_for(1, 8192, 12, pipeline=1)
    assert not kda.pipelined_for(1, 131072, 4, pipeline=1)  # split chains instead
    assert not kda.pipelined_for(1, 8192, 32, chain_segments=4, pipeline=1)
