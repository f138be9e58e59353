"""Arbitrary-precision brute force of the KDA recurrence, tiny inputs only.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

This is a second, independent route to the same numbers as the C oracle.
Instead of the rank-1 update loop it forms the explicit K x K transition of
every token,

    A_t = (I - b_t k_t k_t^T) Diag(exp(a_t)),

and evaluates every state from the unrolled closed form of the recurrence
(gated delta rule with per-channel decay; "What is Kimi Delta Attention
(KDA)", kongchang.com/en, and "¿Qué es la atención Kimi Delta…", 7minutos.es):

    S_t = A_t ... A_1 S_0 + sum_{j<=t} (A_t ... A_{j+1}) b_j k_j v_j^T
    o_t = scale * S_t^T q_t

in mpmath at 40 significant digits.  Cost is O(T^2 K^3) products, so keep
K, V <= 8 and T <= 16.
"""
from __future__ import annotations

import mpmath as mp
import numpy as np

DIGITS = 40
EPS = mp.mpf("1e-6")


def _bf16_to_float(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _gate(g, A_log, dt_bias, lb):
    x = g + dt_bias
    sp = mp.log(1 + mp.exp(x)) if x < 50 else x + mp.log(1 + mp.exp(-x))
    a = -mp.exp(A_log) * sp
    return a if a > lb else lb


def run(q_bits, k_bits, v_bits, g_bits, beta_bits, scale, A_log, dt_bias, lower_bound,
        initial_state=None):
    """Single-sequence brute force.  Shapes: q,k,g [T,H,K]; v [T,H,V];
    beta [T,H] (uint16 bf16 bit patterns); A_log [H]; dt_bias [H,K];
    initial_state [H,K,V] or None.  Returns (out [T,H,V], final [H,K,V]) as
    float64 arrays rounded from 40-digit values."""
    mp.mp.dps = DIGITS
    q = _bf16_to_float(np.asarray(q_bits))
    k = _bf16_to_float(np.asarray(k_bits))
    v = _bf16_to_float(np.asarray(v_bits))
    g = _bf16_to_float(np.asarray(g_bits))
    be = _bf16_to_float(np.asarray(beta_bits))
    T, H, K = q.shape
    V = v.shape[-1]
    scale = mp.mpf(float(np.float32(scale)))
    lb = mp.mpf(float(np.float32(lower_bound)))
    out = np.zeros((T, H, V))
    fin = np.zeros((H, K, V))
    for h in range(H):
        A_list, w_list, qn_list = [], [], []
        for t in range(T):
            kv = [mp.mpf(float(x)) for x in k[t, h]]
            qv = [mp.mpf(float(x)) for x in q[t, h]]
            nk = mp.sqrt(mp.fsum(x * x for x in kv) + EPS)
            nq = mp.sqrt(mp.fsum(x * x for x in qv) + EPS)
            kh = mp.matrix([x / nk for x in kv])
            qh = mp.matrix([x / nq for x in qv])
            bet = mp.mpf(float(be[t, h]))
            if mp.isinf(bet):
                b = mp.mpf(1) if bet > 0 else mp.mpf(0)
            else:
                b = 1 / (1 + mp.exp(-bet))
            dec = [mp.exp(_gate(mp.mpf(float(g[t, h, d])), mp.mpf(float(np.float32(A_log[h]))),
                                mp.mpf(float(np.float32(dt_bias[h, d]))), lb)) for d in range(K)]
            A = (mp.eye(K) - b * (kh * kh.T)) * mp.diag(dec)
            vv = mp.matrix([[mp.mpf(float(x)) for x in v[t, h]]])  # 1 x V
            A_list.append(A)
            w_list.append(b * (kh * vv))  # K x V injection b k v^T
            qn_list.append(qh)
        S0 = mp.zeros(K, V)
        if initial_state is not None:
            S0 = mp.matrix([[mp.mpf(float(initial_state[h][i][j])) for j in range(V)] for i in range(K)])
        S = S0
        for t in range(T):
            # S_t from the unrolled sum, not from S_{t-1}
            P = mp.eye(K)
            acc = mp.zeros(K, V)
            for j in range(t, -1, -1):
                acc += P * w_list[j]
                P = P * A_list[j]
            S = P * S0 + acc
            o = scale * (S.T * qn_list[t])
            for j in range(V):
                out[t, h, j] = float(o[j])
        for i in range(K):
            for j in range(V):
                fin[h, i, j] = float(S[i, j])
    return out, fin
