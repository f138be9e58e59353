"""The value range the fp16 matrix-core operands impose, derived and pinned on the CPU.

The GPU path hands the chunk quantities W, Kbar, Qg, A_qk and T = (I + A_kk)^-1,
the pseudo-values U and Ut = U - W S, and the state S to the matrix cores as
fp16 (largest finite value 65504).  The bounds below say which of them can grow
with the inputs, and how far, so that the public header can state a safe input
scale.  Per (sequence, head), for a value column j (s_j is column j of the
K x V state), with b in [0, 1], decays <= 1 and unit-norm keys and queries:

1. |W|, |Kbar|, |Qg|, |A_qk|, |T| <= 1 entrywise.  Row i of W is the linear
   response of the pseudo-value u_i to the entering state, and that state only
   passes through contractions (I - b k k^T) Diag(e^a) before k_i reads it; T
   is the response to a unit write, for the same reason; the others are
   products of unit vectors and factors <= 1.
2. The delta rule replaces the component of s_j along the written key k by a
   convex combination of its old value and v[j], and leaves the orthogonal
   part alone, so |s_j'|^2 <= |s_j|^2 + v[j]^2 and, over the tokens so far,
       |S[., j]| <= |s_j|_2 <= sqrt(|s_j(0)|_2^2 + sum_t v_t[j]^2).
3. Each pseudo-value u_t[j] = b (v_t[j] - k.(D s_j)) obeys
       |u_t[j]| <= |v_t[j]| + |s_j|_2 (entering token t);
   U is the same from a zero state at the chunk start.
The bounds are attained: keys chosen orthogonal to the current state make (2)
an equality at every step, and a key along the state with the opposite value
makes (3) one.  They are checked here against the fp64 chunk model
(tests/chunked_model.py) on random inputs over the whole lower-bound range and
on those two constructions.
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from tests.chunked_model import _chunk_wy, chunked_forward

K = V = 128
EPS = 1e-6


def _chunks_of(w, bb, h, s0, s1, C=64):
    q, k, v, g, be = (t.double().numpy() for t in (w.q, w.k, w.v, w.g, w.beta))
    A_log = w.A_log.double().numpy()
    dtb = w.dt_bias.double().numpy()
    for c0 in range(s0, s1, C):
        c1 = min(c0 + C, s1)
        yield c0, c1, _chunk_wy(q[bb, c0:c1, h], k[bb, c0:c1, h], v[bb, c0:c1, h], g[bb, c0:c1, h],
                                be[bb, c0:c1, h], A_log[h], dtb[h], float(np.float32(w.lower_bound)),
                                with_inverse=True)


def _check_bounds(w):
    """Walk every chunk of every (sequence, head) with the chunk model and check bounds 1-3.
    Returns the largest ratio of a state / pseudo-value entry to its bound."""
    v = w.v.double().numpy()
    worst = 0.0
    B, T, H = w.B, w.T, w.H
    for bb in range(B):
        for h in range(H):
            S = np.zeros((K, V)) if w.initial_state is None else w.initial_state[bb, h].double().numpy().copy()
            sq = (S * S).sum(0)  # running bound^2 per column: |s_j(0)|^2 + sum v^2
            for c0, c1, (Qg, Mqk, Wc, Uc, Kbar, gn, Tm) in _chunks_of(w, bb, h, 0, T):
                for name, X in (("W", Wc), ("Kbar", Kbar), ("Qg", Qg), ("A_qk", Mqk), ("T", Tm)):
                    assert np.abs(X).max() <= 1 + 1e-9, (name, np.abs(X).max())
                vv = v[bb, c0:c1, h]
                # U: pseudo-values from a zero state at the chunk start
                pre = np.sqrt(np.concatenate([np.zeros((1, V)), np.cumsum(vv * vv, 0)[:-1]]))
                ub = np.abs(vv) + pre
                assert (np.abs(Uc) <= ub * (1 + 1e-9) + 1e-12).all()
                # Ut from the entering state, token by token within the chunk
                Ut = Uc - Wc @ S
                run = sq[None, :] + np.concatenate([np.zeros((1, V)), np.cumsum(vv * vv, 0)[:-1]])
                utb = np.abs(vv) + np.sqrt(run)
                assert (np.abs(Ut) <= utb * (1 + 1e-9) + 1e-12).all()
                worst = max(worst, float((np.abs(Ut) / np.maximum(utb, 1e-300)).max()))
                S = gn[:, None] * S + Kbar.T @ Ut
                sq = sq + (vv * vv).sum(0)
                colnorm = np.sqrt((S * S).sum(0))
                assert (colnorm <= np.sqrt(sq) * (1 + 1e-9) + 1e-12).all()
                worst = max(worst, float((colnorm / np.maximum(np.sqrt(sq), 1e-300)).max()))
    return worst


@pytest.mark.parametrize("lb,g_mean,beta_std", [(-5.0, 0.0, 1.0), (-1.0, -2.0, 3.0), (0.0, 0.0, 1.0),
                                                (-5.0, -8.0, 1.0)])
def test_bounds_hold_on_random_inputs(lb, g_mean, beta_std):
    w = W.make("range_bounds", 2, 150, 2, 9100, lower_bound=lb, g_mean=g_mean, beta_std=beta_std,
               init="fp32", final="fp32")
    w.initial_state = w.initial_state * 30.0  # a state far from the inputs' own scale
    ratio = _check_bounds(w)
    assert 0 < ratio <= 1 + 1e-9


def _adversarial(T, kind, seed=9101):
    """No decay (lb = 0), b = 1, v[j] = 1 on every token and column.  "grow": every key is
    orthogonal to the current state's column 0, so |s_0| grows by exactly 1 in square per
    token; "read": the same for T - 1 tokens, then a key along column 0 of the state and
    v = -1, so that |u[0]| = 1 + |s_0| exactly."""
    rng = np.random.default_rng(seed)
    keys = np.zeros((T, K))
    s = np.zeros(K)  # column 0 of the state
    for t in range(T):
        if kind == "read" and t == T - 1:
            kk = s / np.linalg.norm(s)
        else:
            kk = rng.standard_normal(K)
            if t > 0:
                kk -= s * (kk @ s) / (s @ s)
            kk /= np.linalg.norm(kk)
        keys[t] = kk
        val = -1.0 if (kind == "read" and t == T - 1) else 1.0
        s = s + kk * (val - kk @ s)  # b = 1, no decay
    vals = np.ones((T, V))
    if kind == "read":
        vals[-1] = -1.0
    t64 = lambda a: torch.from_numpy(a)
    q = t64(rng.standard_normal((1, T, 1, K)))
    w = W.Workload("adv", 1, T, 1, K, V, q, t64(keys[None, :, None, :].copy()), t64(vals[None, :, None, :].copy()),
                   torch.zeros((1, T, 1, K), dtype=torch.float64),
                   torch.full((1, T, 1), math.inf, dtype=torch.float64),
                   torch.zeros(1), torch.zeros((1, K)), 0.0, 1.0, torch.zeros((1, 1, K, V), dtype=torch.float64),
                   torch.float32, None, [T])
    return w


def test_state_bound_is_attained():
    # keys orthogonal to the state: |s_0|_2 = sqrt(T) after T unit writes, the bound exactly
    T = 150
    w = _adversarial(T, "grow")
    _, fin = chunked_forward(w)
    n0 = np.linalg.norm(fin[0, 0][:, 0])
    assert abs(n0 - math.sqrt(T * (1 - EPS / (1 + EPS)))) <= 1e-6 * math.sqrt(T), n0
    assert _check_bounds(w) >= 1 - 1e-6


def test_pseudo_value_bound_is_attained():
    # then a key along the state with value -1: |u| = 1 + |s_0|_2
    T = 130
    w = _adversarial(T, "read")
    assert _check_bounds(w) >= 1 - 1e-6


def test_safe_scale_quoted_in_header():
    # The header's examples: |v| <= 160 and |S_0| <= 100 up to 131072 tokens, |v| <= 1500 and
    # |S_0| <= 1000 up to 1024 tokens, keep every bounded quantity below fp16's 65504.
    for vmax, smax, T in ((160.0, 100.0, 131072), (1500.0, 1000.0, 1024)):
        state = math.sqrt(K * smax ** 2 + T * vmax ** 2)
        assert state + vmax < 65504.0
    with open("include/kda.h") as f:
        text = f.read()
    assert "|v| <= 160 and |initial_state| <= 100" in text and "|v| <= 1500" in text
