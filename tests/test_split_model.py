"""The split-chain decomposition the library uses for long sequences (every
segment's affine state map, an ordered scan of the maps, each segment re-run
from its entering state), written out in fp64 numpy (tests/chunked_model.py),
reaches the oracle's token recurrence: the chunk map is affine, so the split is
exact up to rounding.  CPU only."""
import numpy as np
import pytest

import workloads as W
from tests.chunked_model import _bf16_to_f64, _chunk_wy, split_forward
from tests.parity import run_oracle


@pytest.mark.parametrize("B,T,C,segs,init", [
    (1, 150, 8, 4, "fp32"),     # ragged last chunk, 19 chunks in segments of 5
    (2, 97, 16, 3, None),       # two batch rows, no initial state
    (1, 64, 8, 8, "fp32"),      # one chunk per segment
    (1, 40, 8, 1, "fp32"),      # a single segment: the plain chunked form
])
def test_split_decomposition_equals_oracle(B, T, C, segs, init):
    w = W.make("splitmodel", B, T, 2, 700 + T + segs, K=16, V=8, init=init, g_mean=-1.0)
    ro, rf = run_oracle(w)
    so, sf = split_forward(w, segs, C)
    assert np.abs(so - ro).max() <= 1e-11, np.abs(so - ro).max()
    assert np.abs(sf - rf).max() <= 1e-11, np.abs(sf - rf).max()


def test_split_with_a_wrong_composition_order_fails():
    # composing the segment maps last-first is a plausible slip: it must miss the oracle's
    # final state by far, while the in-order composition meets it
    w = W.make("splitmodel", 1, 120, 1, 790, K=8, V=8, init="fp32", g_mean=-0.5)
    ro, rf = run_oracle(w)
    q, k, v, g, be = (_bf16_to_f64(t) for t in (w.q, w.k, w.v, w.g, w.beta))
    A_log, dtb = w.A_log.double().numpy()[0], w.dt_bias.double().numpy()[0]
    maps = []
    for s0 in range(0, 15, 5):            # 15 chunks of 8 tokens, 3 segments of 5 chunks
        M, N = np.eye(8), np.zeros((8, 8))
        for c in range(s0, s0 + 5):
            sl = slice(8 * c, 8 * c + 8)
            _, _, Wc, Uc, Kbar, gn = _chunk_wy(q[0, sl, 0], k[0, sl, 0], v[0, sl, 0], g[0, sl, 0],
                                              be[0, sl, 0], A_log, dtb, float(w.lower_bound))
            M = gn[:, None] * M + Kbar.T @ (-Wc @ M)
            N = gn[:, None] * N + Kbar.T @ (Uc - Wc @ N)
        maps.append((M, N))
    good = bad = w.initial_state[0, 0].double().numpy()
    for M, N in maps:
        good = M @ good + N
    for M, N in reversed(maps):
        bad = M @ bad + N
    assert np.abs(good - rf[0, 0]).max() <= 1e-11
    assert np.abs(bad - rf[0, 0]).max() > 1e-3
