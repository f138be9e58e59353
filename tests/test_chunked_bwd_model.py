"""The chunked gradient (tests/chunked_bwd_model.py: the decomposition the GPU
backward follows) against the oracle's token-by-token gradient, on the CPU.
In exact arithmetic the two are the same function, so agreement to ~1e-12 pins
both: the oracle's reverse recurrence and the chunk algebra (forward states,
the backward state chain, and the per-chunk gradient through the UT inverse,
the decayed Gram matrices and the gate)."""
import numpy as np
import pytest

import oracle
from tests.chunked_bwd_model import chunked_backward


def _case(B, T, H, K, V, seed, N=None, lb=-3.0):
    rng = np.random.default_rng(seed)
    N = N or B
    return dict(q=rng.standard_normal((B, T, H, K)), k=rng.standard_normal((B, T, H, K)),
                v=rng.standard_normal((B, T, H, V)), g=rng.standard_normal((B, T, H, K)) * 2.0,
                beta=rng.standard_normal((B, T, H)), A_log=rng.uniform(-1.0, 0.5, H),
                dt_bias=rng.standard_normal((H, K)) * 0.5, initial_state=rng.standard_normal((N, H, K, V)),
                d_out=rng.standard_normal((B, T, H, V)), d_final=rng.standard_normal((N, H, K, V)), lb=lb)


@pytest.mark.parametrize("B,T,H,K,V,C,cu,lb", [
    (2, 37, 2, 8, 6, 8, None, -3.0),          # ragged last chunk, K != V
    (1, 150, 2, 16, 16, 64, None, -5.0),      # three 64-token chunks
    (1, 90, 1, 8, 8, 16, [0, 20, 20, 90], -1.0),  # packed, with an empty sequence
    (1, 70, 1, 4, 4, 64, None, 0.0),          # no decay
])
def test_chunked_gradient_matches_oracle(B, T, H, K, V, C, cu, lb):
    N = len(cu) - 1 if cu else B
    x = _case(B, T, H, K, V, seed=T + K, N=N, lb=lb)
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"], 0.4, x["A_log"], x["dt_bias"], lb, x["d_out"])
    ref = oracle.bwd(*args, d_final=x["d_final"], initial_state=x["initial_state"], cu_seqlens=cu)
    got = chunked_backward(*args, d_final=x["d_final"], initial_state=x["initial_state"], cu_seqlens=cu, C=C)
    for name in ref:
        err = np.abs(ref[name] - got[name]).max()
        assert err <= 1e-11 * max(1.0, np.abs(ref[name]).max()), (name, err)


@pytest.mark.parametrize("segments", [2, 3, 13])
def test_split_chains_match_oracle(segments):
    # the split chains of the GPU plan (forward maps composed in order; reverse chains from a
    # zero gradient composed with the transposed forward maps, last segment first) give the
    # same gradient: 13 chunks of 8 tokens (the last ragged) in 2, 3 and 13 segments
    B, T, H, K, V, C = 2, 8 * 12 + 5, 2, 8, 6, 8
    x = _case(B, T, H, K, V, seed=977, lb=-2.0)
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"], 0.4, x["A_log"], x["dt_bias"], -2.0, x["d_out"])
    ref = oracle.bwd(*args, d_final=x["d_final"], initial_state=x["initial_state"])
    got = chunked_backward(*args, d_final=x["d_final"], initial_state=x["initial_state"], C=C,
                           segments=segments)
    for name in ref:
        err = np.abs(ref[name] - got[name]).max()
        assert err <= 1e-11 * max(1.0, np.abs(ref[name]).max()), (name, err)
