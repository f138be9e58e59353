"""Chunked (WY / UT) gradient of KDA in plain numpy fp64 -- the plan the GPU
backward follows, written out so that it can be checked against the oracle's
token-by-token gradient (oracle/kda_oracle_bwd.c) before any kernel runs.

Nothing here is shared with the oracle or the HIP library.  Per (sequence,
head) it runs the same three passes as the GPU:

1. forward state chain: the state h_c entering every chunk;
2. backward state chain, last chunk first, with dS the gradient of the
   state leaving the chunk:
       dUt  = scale A_qk^T dO + Kbar dS
       dS  <- Diag(exp(G_n)) dS - W^T dUt + scale Qg^T dO
   (dh_c = the dS entering this step, the gradient of the state leaving chunk c);
3. per chunk, independently, with S = h_c, dS' = dh_c and dUt:
       Y   = V - (gamma * Khat) S,   Ut = T Diag(b) Y,   Z = T^T dUt
       dQg = scale dO S^T,   Zw = -Z S^T,   dKbar = Ut dS'^T
       dA_qk = scale dO Ut^T (j <= i),   dA_kk = -Z Ut^T (j < i)
   then the Gram matrices' gradients through the per-channel decays, and the
   chain rule down to q, k, v, g, beta, A_log and dt_bias.

T = (I + Diag(b) M)^-1 with M the strictly lower decayed key Gram, and
U - W S = T Diag(b) Y, so W and U are never needed apart: the gradient of
(I + Diag(b) M) is -T^T dT T^T = -Z Ut^T.

With ``segments`` the two state chains are split as the GPU splits them: the
chunks of a sequence are cut into segments of ceil(chunks / segments) chunks;
the forward composes every segment's affine map S -> M S + N (M from S = I
with U = 0, N from S = 0) in order; the backward runs every segment's reverse
chain from a zero gradient (N'), composes D_s = M_s^T D_{s+1} + N'_s from the
last segment to the first, and runs every segment again from the gradient
leaving it.  Both are the unsplit chains in exact arithmetic.
"""
from __future__ import annotations

import numpy as np

EPS = 1e-6


def _softplus(x):
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def _chunk_prep(q, k, g, be, A, dtb, lb):
    """fp64 chunk quantities: qhat, khat, rq, rk, b, z (unclamped gate), G, M, A_qk, T."""
    rq = 1.0 / np.sqrt((q * q).sum(-1, keepdims=True) + EPS)
    rk = 1.0 / np.sqrt((k * k).sum(-1, keepdims=True) + EPS)
    qn, kn = q * rq, k * rk
    b = 1.0 / (1.0 + np.exp(-be))
    z = -np.exp(A) * _softplus(g + dtb)
    a = np.maximum(lb, z)
    G = np.cumsum(a, axis=0)
    n = q.shape[0]
    low = np.tril(np.ones((n, n), dtype=bool), -1)
    lowd = low | np.eye(n, dtype=bool)
    E = np.where(lowd[:, :, None], np.exp(np.minimum(G[:, None, :] - G[None, :, :], 0.0)), 0.0)
    M = np.einsum("id,jd,ijd->ij", kn, kn, E) * low
    Aqk = np.einsum("id,jd,ijd->ij", qn, kn, E) * lowd
    T = np.linalg.inv(np.eye(n) + b[:, None] * M)
    return dict(qn=qn, kn=kn, rq=rq, rk=rk, b=b, z=z, G=G, M=M, Aqk=Aqk, T=T, E=E, low=low, lowd=lowd)


def _segments(n, segments):
    """Chunk index ranges of the segments of an n-chunk chain (one range when unsplit)."""
    if not segments or segments < 2 or n < 2:
        return [range(n)]
    segc = -(-n // min(segments, n))
    return [range(s, min(s + segc, n)) for s in range(0, n, segc)]


def chunked_backward(q, k, v, g, beta, scale, A_log, dt_bias, lb, d_out, d_final=None, initial_state=None,
                     cu_seqlens=None, C: int = 64, segments=None):
    """Gradient of the forward pass, computed chunk by chunk.  fp64 numpy inputs as
    oracle.bwd takes them; returns the same dict of arrays."""
    B, T_, H, K = q.shape
    V = v.shape[-1]
    seqs = [(b, 0, T_) for b in range(B)] if cu_seqlens is None else \
        [(0, cu_seqlens[n], cu_seqlens[n + 1]) for n in range(len(cu_seqlens) - 1)]
    N = len(seqs)
    res = {"dq": np.zeros_like(q), "dk": np.zeros_like(k), "dv": np.zeros_like(v), "dg": np.zeros_like(g),
           "dbeta": np.zeros_like(beta), "d_initial": np.zeros((N, H, K, V)), "dA_log": np.zeros(H),
           "ddt_bias": np.zeros((H, K))}
    for n, (bb, s0, s1) in enumerate(seqs):
        for h in range(H):
            A, dtb = A_log[h], dt_bias[h]
            chunks = [(c0, min(c0 + C, s1)) for c0 in range(s0, s1, C)]
            preps, wy = [], []
            for c0, c1 in chunks:
                p = _chunk_prep(q[bb, c0:c1, h], k[bb, c0:c1, h], g[bb, c0:c1, h], beta[bb, c0:c1, h], A, dtb, lb)
                gam = np.exp(p["G"])
                gn = gam[-1]
                W = p["T"] @ (p["b"][:, None] * gam * p["kn"])
                U = p["T"] @ (p["b"][:, None] * v[bb, c0:c1, h])
                Kbar = np.exp(p["G"][-1][None, :] - p["G"]) * p["kn"]
                preps.append(p)
                wy.append((W, U, Kbar, gam * p["qn"], gn))

            def fstep(S, ci, linear=False):
                W, U, Kbar, _, gn = wy[ci]
                return gn[:, None] * S + Kbar.T @ ((0.0 if linear else U) - W @ S)

            def rstep(dS, ci):
                W, _, Kbar, Qg, gn = wy[ci]
                c0, c1 = chunks[ci]
                dO = d_out[bb, c0:c1, h]
                dUt = scale * preps[ci]["Aqk"].T @ dO + Kbar @ dS
                return gn[:, None] * dS - W.T @ dUt + scale * Qg.T @ dO, dUt

            segs = _segments(len(chunks), segments)
            # 1. forward states: the state entering every segment (composed maps), then
            # every chunk's from it
            S = np.zeros((K, V)) if initial_state is None else initial_state[n, h].copy()
            maps, s_in = [], []
            for seg in segs:
                M, Nn = np.eye(K), np.zeros((K, V))
                for ci in seg:
                    M, Nn = fstep(M, ci, linear=True), fstep(Nn, ci)
                maps.append(M)
                s_in.append(S)
                S = M @ S + Nn
            hs = [None] * len(chunks)
            for seg, S in zip(segs, s_in):
                for ci in seg:
                    hs[ci] = S.copy()
                    S = fstep(S, ci)
            # 2. backward chain: the gradient leaving every segment (reverse maps: M_s^T
            # and the chain from zero), then every chunk's from it
            dS = np.zeros((K, V)) if d_final is None else d_final[n, h].copy()
            d_leave = [None] * len(segs)
            for si in range(len(segs) - 1, -1, -1):
                d_leave[si] = dS
                off = np.zeros((K, V))
                for ci in reversed(segs[si]):
                    off, _ = rstep(off, ci)
                dS = maps[si].T @ dS + off
            res["d_initial"][n, h] = dS
            dhs, dUts = [None] * len(chunks), [None] * len(chunks)
            for si, seg in enumerate(segs):
                dS = d_leave[si]
                for ci in reversed(seg):
                    dhs[ci] = dS.copy()
                    dS, dUts[ci] = rstep(dS, ci)
            # 3. per chunk
            for ci, (c0, c1) in enumerate(chunks):
                p = preps[ci]
                qn, kn, b, G, T, M, Aqk = p["qn"], p["kn"], p["b"], p["G"], p["T"], p["M"], p["Aqk"]
                vv, dO = v[bb, c0:c1, h], d_out[bb, c0:c1, h]
                S, dSp, dUt = hs[ci], dhs[ci], dUts[ci]
                gam = np.exp(G)
                gn = gam[-1]
                Kbar = np.exp(G[-1][None, :] - G) * kn
                Y = vv - (gam * kn) @ S
                Ut = T @ (b[:, None] * Y)
                Z = T.T @ dUt
                dQg = scale * dO @ S.T
                Zw = -Z @ S.T
                dKbar = Ut @ dSp.T
                dGn = gn * (S * dSp).sum(1)
                dAqk = scale * (dO @ Ut.T) * p["lowd"]
                dAkk = -(Z @ Ut.T) * p["low"]
                dM = b[:, None] * dAkk
                db = (dAkk * M).sum(1)
                # Gram matrices through the decays: P[i,j] = sum_d x_i y_j exp(G_i - G_j)
                E = p["E"]
                RxM = np.einsum("ij,jd,ijd->id", dM, kn, E)
                RxA = np.einsum("ij,jd,ijd->id", dAqk, kn, E)
                Ry = np.einsum("ij,id,ijd->jd", dM, kn, E) + np.einsum("ij,id,ijd->jd", dAqk, qn, E)
                dkn = RxM + Ry
                dqn = RxA.copy()
                dG = kn * RxM + qn * RxA - kn * Ry
                # Y = V - (gamma * Khat) S and Diag(b) Y
                dv = b[:, None] * Z
                db += (Z * vv).sum(1) + (Zw * gam * kn).sum(1)
                dkn += b[:, None] * gam * Zw
                dG += b[:, None] * gam * kn * Zw
                # Qg = gamma * qhat, Kbar = exp(G_n - G) * khat
                dqn += gam * dQg
                dG += gam * qn * dQg
                dkn += np.exp(G[-1][None, :] - G) * dKbar
                dG -= Kbar * dKbar
                dGn += (Kbar * dKbar).sum(0)
                dG[-1] += dGn
                da = np.cumsum(dG[::-1], axis=0)[::-1]
                # gate, norms, beta
                x = g[bb, c0:c1, h] + dtb
                free = p["z"] > lb
                dx = np.where(free, da * (-np.exp(A)) / (1.0 + np.exp(-x)), 0.0)
                res["dg"][bb, c0:c1, h] = dx
                res["ddt_bias"][h] += dx.sum(0)
                res["dA_log"][h] += np.where(free, da * p["z"], 0.0).sum()
                qq, kk = q[bb, c0:c1, h], k[bb, c0:c1, h]
                rq, rk = p["rq"], p["rk"]
                res["dq"][bb, c0:c1, h] = rq * dqn - rq ** 3 * (qq * dqn).sum(-1, keepdims=True) * qq
                res["dk"][bb, c0:c1, h] = rk * dkn - rk ** 3 * (kk * dkn).sum(-1, keepdims=True) * kk
                res["dv"][bb, c0:c1, h] = dv
                res["dbeta"][bb, c0:c1, h] = db * b * (1.0 - b)
    return res
