"""GPU parity on seeded random shapes, against the fp64 oracle.

Each case draws, from its own seed, a batch size, a length, a head count (up to
40 (sequence, head) chains, so that both the one-block and the two-block chain
kernels run), packed or fixed-length rows (packed lengths include empty and
one-token sequences), the presence and dtype of the initial and final states,
the lower bound, the mean of the gate input and, for fixed-length rows, a
forced chain split.  Every case must meet the same tolerances as the fixed
workloads: bf16 outputs max-abs 2e-2 and relative RMS 5e-3, fp32 states 1e-3,
bf16 states 5e-3.
"""
import numpy as np
import pytest

import workloads as W
from tests.parity import compare, run_gpu, run_oracle, say, to_np

pytestmark = pytest.mark.gpu

N_CASES = 24


def _draw(i):
    r = np.random.Generator(np.random.PCG64(8000 + i))
    H = int(r.integers(1, 13))
    packed = bool(r.random() < 0.4)
    init = [None, "fp32", "bf16"][int(r.integers(0, 3))]
    final = [None, "fp32", "bf16"][int(r.integers(0, 3))]
    lb = float([-5.0, -3.0, -1.0, 0.0][int(r.integers(0, 4))])
    g_mean = float(r.uniform(-4.0, 1.0))
    segs = 0
    if packed:
        n = int(r.integers(1, max(2, 40 // H) + 1))
        lens = [int(x) for x in r.choice([0, 1, 2, 63, 64, 65, 100, 127, 128, 129, 200, 300], size=n)]
        if sum(lens) == 0:
            lens[0] = 5
        return dict(B=1, T=sum(lens), H=H, seqlens=lens, init=init, final=final, lb=lb, g_mean=g_mean, segs=0)
    B = int(r.integers(1, max(2, 40 // H) + 1))
    T = int(r.integers(1, 700))
    if r.random() < 0.3 and T > 64:
        segs = int(r.integers(2, 6))
    return dict(B=B, T=T, H=H, seqlens=None, init=init, final=final, lb=lb, g_mean=g_mean, segs=segs)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_matches_oracle(i):
    c = _draw(i)
    say("case random %d: %s" % (i, c))
    w = W.make("random%d" % i, c["B"], c["T"], c["H"], 8100 + i, lower_bound=c["lb"], g_mean=c["g_mean"],
               init=c["init"], final=c["final"], seqlens=c["seqlens"])
    out, fin = run_gpu(w, chain_segments=c["segs"])
    ro, rf = run_oracle(w)
    res = compare(to_np(out), ro, to_np(fin), None if fin is None else rf, w.final_state_dtype,
                  "random %d" % i)
    say("  %s" % res)
