"""Chunk-parallel (WY / UT) form of KDA in plain numpy fp64 -- a second route.

Used only by the tests, to pin the token-recurrence oracle: in exact
arithmetic the chunked form below reaches the same outputs and states, so
agreement to ~1e-12 checks the oracle's decay order, delta write and output
timing through an independent derivation.  Nothing here is shared with the
oracle or the HIP library.

Within a chunk of n tokens entering with state S0 (K x V), with cumulative
log-decays G_i = sum_{t<=i} a_t (per channel):
    A[i,j]  = b_i sum_d k_i[d] k_j[d] exp(G_i[d] - G_j[d])        (j < i)
    M[i,j]  =     sum_d q_i[d] k_j[d] exp(G_i[d] - G_j[d])        (j <= i)
    Ut      = (I + A)^-1 (Diag(b) V - Diag(b) (exp(G) * K) S0)
    O       = scale (exp(G) * Q) S0 + scale M Ut
    S_n     = Diag(exp(G_n)) S0 + (exp(G_n - G) * K)^T Ut
(Yang et al., "Parallelizing Linear Transformers with the Delta Rule over
Sequence Length", with the scalar decay replaced by a per-channel one.)
"""
from __future__ import annotations

import numpy as np

EPS = 1e-6


def _bf16_to_f64(t) -> np.ndarray:
    return t.double().numpy()


def _softplus(x):
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def chunked_forward(w, C: int = 64):
    """fp64 chunked forward of a workloads.Workload; returns (out, final)."""
    q, k, v, g, be = (_bf16_to_f64(t) for t in (w.q, w.k, w.v, w.g, w.beta))
    B, T, H, K = q.shape
    V = v.shape[-1]
    A_log = w.A_log.double().numpy()
    dtb = w.dt_bias.double().numpy()
    lb = float(np.float32(w.lower_bound))
    scale = float(np.float32(w.scale))
    if w.cu_seqlens is None:
        seqs = [(b, 0, T) for b in range(B)]
    else:
        cu = w.cu_seqlens.tolist()
        seqs = [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]
    out = np.zeros((B, T, H, V))
    fin = np.zeros((len(seqs), H, K, V))
    for n, (bb, s0, s1) in enumerate(seqs):
        for h in range(H):
            S = np.zeros((K, V)) if w.initial_state is None else w.initial_state[n, h].double().numpy().copy()
            for c0 in range(s0, s1, C):
                c1 = min(c0 + C, s1)
                qq, kk, vv = q[bb, c0:c1, h], k[bb, c0:c1, h], v[bb, c0:c1, h]
                qn = qq / np.sqrt((qq * qq).sum(-1, keepdims=True) + EPS)
                kn = kk / np.sqrt((kk * kk).sum(-1, keepdims=True) + EPS)
                b = 1.0 / (1.0 + np.exp(-be[bb, c0:c1, h]))
                a = np.maximum(lb, -np.exp(A_log[h]) * _softplus(g[bb, c0:c1, h] + dtb[h]))
                G = np.cumsum(a, axis=0)
                n_ = c1 - c0
                low = np.tril(np.ones((n_, n_), dtype=bool), -1)
                diff = G[:, None, :] - G[None, :, :]
                E = np.where((low | np.eye(n_, dtype=bool))[:, :, None], np.exp(np.minimum(diff, 0.0)), 0.0)
                A = b[:, None] * np.einsum("id,jd,ijd->ij", kn, kn, E) * low
                Mqk = np.einsum("id,jd,ijd->ij", qn, kn, E)
                rhs = b[:, None] * vv - (b[:, None] * np.exp(G) * kn) @ S
                Ut = np.linalg.solve(np.eye(n_) + A, rhs)
                out[bb, c0:c1, h] = scale * ((np.exp(G) * qn) @ S + Mqk @ Ut)
                S = np.exp(G[-1])[:, None] * S + (np.exp(G[-1][None, :] - G) * kn).T @ Ut
            fin[n, h] = S
    return out, fin


def _chunk_wy(qq, kk, vv, gg, bb, A_log_h, dtb_h, lb, with_inverse=False):
    """WY quantities of one chunk: (Qg, Mqk, W, U, Kbar, gn) with
    Ut = U - W S, O = Qg S + Mqk Ut (unscaled), S_next = Diag(gn) S + Kbar^T Ut;
    with_inverse also returns T = (I + A)^-1 last."""
    qn = qq / np.sqrt((qq * qq).sum(-1, keepdims=True) + EPS)
    kn = kk / np.sqrt((kk * kk).sum(-1, keepdims=True) + EPS)
    b = 1.0 / (1.0 + np.exp(-bb))
    a = np.maximum(lb, -np.exp(A_log_h) * _softplus(gg + dtb_h))
    G = np.cumsum(a, axis=0)
    n_ = len(b)
    low = np.tril(np.ones((n_, n_), dtype=bool), -1)
    diff = G[:, None, :] - G[None, :, :]
    E = np.where((low | np.eye(n_, dtype=bool))[:, :, None], np.exp(np.minimum(diff, 0.0)), 0.0)
    A = b[:, None] * np.einsum("id,jd,ijd->ij", kn, kn, E) * low
    Mqk = np.einsum("id,jd,ijd->ij", qn, kn, E)
    Tm = np.linalg.inv(np.eye(n_) + A)
    W = Tm @ (b[:, None] * np.exp(G) * kn)
    U = Tm @ (b[:, None] * vv)
    Kbar = np.exp(G[-1][None, :] - G) * kn
    if with_inverse:
        return np.exp(G) * qn, Mqk, W, U, Kbar, np.exp(G[-1]), Tm
    return np.exp(G) * qn, Mqk, W, U, Kbar, np.exp(G[-1])


def split_forward(w, segs: int, C: int = 64):
    """fp64 forward with every sequence's chunk chain cut into ``segs`` segments of
    ceil(chunks / segs) chunks (fixed-length batches): each segment's affine map
    S -> M S + N (M from S = I with U = 0, N from S = 0), the maps composed in
    order from the initial state, then every segment re-run from its entering
    state.  In exact arithmetic this equals the unsplit forward."""
    assert w.cu_seqlens is None
    q, k, v, g, be = (_bf16_to_f64(t) for t in (w.q, w.k, w.v, w.g, w.beta))
    B, T, H, K = q.shape
    V = v.shape[-1]
    A_log = w.A_log.double().numpy()
    dtb = w.dt_bias.double().numpy()
    lb = float(np.float32(w.lower_bound))
    scale = float(np.float32(w.scale))
    nc = (T + C - 1) // C
    segc = max(1, (nc + segs - 1) // segs)
    out = np.zeros((B, T, H, V))
    fin = np.zeros((B, H, K, V))
    for bb in range(B):
        for h in range(H):
            chunks = []
            for c in range(nc):
                c0, c1 = c * C, min(c * C + C, T)
                chunks.append((c0, c1, _chunk_wy(q[bb, c0:c1, h], k[bb, c0:c1, h], v[bb, c0:c1, h],
                                                  g[bb, c0:c1, h], be[bb, c0:c1, h], A_log[h], dtb[h], lb)))
            segments = [chunks[i:i + segc] for i in range(0, nc, segc)]
            maps = []
            for seg in segments:   # 1. the map of every segment
                M, N = np.eye(K), np.zeros((K, V))
                for _, _, (Qg, Mqk, Wc, Uc, Kbar, gn) in seg:
                    M = gn[:, None] * M + Kbar.T @ (-Wc @ M)
                    N = gn[:, None] * N + Kbar.T @ (Uc - Wc @ N)
                maps.append((M, N))
            S = np.zeros((K, V)) if w.initial_state is None else w.initial_state[bb, h].double().numpy().copy()
            entering = []
            for M, N in maps:      # 2. the scan
                entering.append(S)
                S = M @ S + N
            fin[bb, h] = S
            for seg, S in zip(segments, entering):   # 3. every segment from its entering state
                for c0, c1, (Qg, Mqk, Wc, Uc, Kbar, gn) in seg:
                    Ut = Uc - Wc @ S
                    out[bb, c0:c1, h] = scale * (Qg @ S + Mqk @ Ut)
                    S = gn[:, None] * S + Kbar.T @ Ut
    return out, fin
