"""The intra-chunk kernel's intermediates, read back from the workspace and
compared chunk by chunk with the fp64 chunk model (tests/chunked_model.py):
-W, Qg, Kbar^T, A_qk, U (fp16, MFMA fragment order) and exp(G_n) (fp32), and
for a packed batch the chunk table the chunk-table kernel writes.

The fragment order is the one the library documents for its workspace: lane
l = r + 16 g of fragment (t, p) holds row 16 t + r and the eight k slots
perm(p, g, j) = 32 p + 4 g + j (j < 4) or 32 p + 16 + 4 g + (j - 4) (j >= 4);
U is stored as [16-column block][row tile][lane][4] with rows 16 t + 4 g + e.
Rows past the end of a ragged chunk hold zeros (no key, no query, b = 0).
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_110_amd as kda
import workloads as W
from tests.chunked_model import _chunk_wy
from tests.parity import say

pytestmark = pytest.mark.gpu

C, K, V = 64, 128, 128


def _align(x, a=256):
    return (x + a - 1) // a * a


def _layout(slots, H, N, packed):
    """Byte offsets of the workspace buffers (the library's order)."""
    per = slots * H
    o = 0
    off = {}
    off["chunk_off"] = o; o = _align(o + (4 * (N + 1) if packed else 0))
    off["seq_order"] = o; o = _align(o + (4 * N if packed else 0))
    for name, elems, size in (("Wf", C * K, 2), ("Qf", C * K, 2), ("Kf", K * C, 2), ("Af", C * C, 2),
                              ("Uf", C * V, 2), ("gn", K, 4)):
        off[name] = o
        o = _align(o + per * elems * size)
    return off


def _perm(p, g, j):
    return 32 * p + 4 * g + j if j < 4 else 32 * p + 16 + 4 * g + (j - 4)


def _rows_cols(n_t, n_p):
    """(row, col) of every element of a [n_t][n_p][64 lane][8] fragment buffer."""
    rows = np.zeros((n_t, n_p, 64, 8), dtype=np.int64)
    cols = np.zeros_like(rows)
    for t in range(n_t):
        for p in range(n_p):
            for lane in range(64):
                r, g = lane & 15, lane >> 4
                for j in range(8):
                    rows[t, p, lane, j] = 16 * t + r
                    cols[t, p, lane, j] = _perm(p, g, j)
    return rows.ravel(), cols.ravel()


W_RC = _rows_cols(4, 4)   # Wf, Qf: [row tile][k-block] -> (token row, channel)
K_RC = _rows_cols(8, 2)   # Kf: [channel tile][token block] -> (channel, token)
A_RC = _rows_cols(4, 2)   # Af: [row tile][column block] -> (token row, token column)


def _unfrag(buf, rc, shape):
    m = np.zeros(shape)
    m[rc[0], rc[1]] = buf
    return m


def _unfrag_u(buf):
    u = np.zeros((C, V))
    b = buf.reshape(8, 4, 64, 4)
    for vb in range(8):
        for t in range(4):
            for lane in range(64):
                r, g = lane & 15, lane >> 4
                u[16 * t + 4 * g: 16 * t + 4 * g + 4, 16 * vb + r] = b[vb, t, lane]
    return u


def _close(got, ref, what, rel=2e-3):
    err = np.abs(got - ref).max()
    tol = rel * max(np.abs(ref).max(), 1e-30)
    assert err <= tol, "%s: max abs error %.3e > %.3e" % (what, err, tol)
    return err / max(np.abs(ref).max(), 1e-30)


@pytest.mark.parametrize("packed", [False, True])
def test_intermediates_match_chunk_model(packed):
    H = 2
    if packed:
        lens = [70, 0, 64, 5, 130]
        w = W.make("inter", 1, sum(lens), H, 7701, lower_bound=-5.0, init=None, final="fp32", seqlens=lens)
        seqs = []
        t0 = 0
        for L in lens:
            seqs.append((0, t0, t0 + L))
            t0 += L
    else:
        w = W.make("inter", 2, 64 * 2 + 17, H, 7702, lower_bound=-5.0, init=None, final="fp32")
        seqs = [(b, 0, w.T) for b in range(w.B)]
    N = len(seqs)
    nc = (w.T + C - 1) // C
    slots = nc + N if packed else w.B * nc
    need = kda.workspace_size(w.B, w.T, H, num_seqs=N)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    wd = w.to("cuda")
    kda.fwd(wd.q, wd.k, wd.v, wd.g, wd.beta, w.scale, None, wd.A_log, wd.dt_bias, w.lower_bound,
            None, None, wd.cu_seqlens, workspace=ws)
    torch.cuda.synchronize()
    host = ws.cpu().numpy()
    off = _layout(slots, H, N, packed)

    def frag(name, dtype, elems, idx):
        a = host[off[name]:].view(dtype)
        return a[idx * elems:(idx + 1) * elems].astype(np.float64)

    # chunk table: first chunk slot of every packed sequence (ceil(len / 64) chunks each)
    first = []
    s = 0
    for (_, a0, a1) in seqs:
        first.append(s)
        s += (a1 - a0 + C - 1) // C if packed else nc
    if packed:
        table = host[off["chunk_off"]:off["chunk_off"] + 4 * (N + 1)].view(np.int32)
        assert table.tolist() == first + [s], (table.tolist(), first + [s])
        order = sorted(host[off["seq_order"]:off["seq_order"] + 4 * N].view(np.int32).tolist())
        assert order == list(range(N))
    q, k, v, g, be = (t.double().numpy() for t in (w.q, w.k, w.v, w.g, w.beta))
    A_log, dtb = w.A_log.double().numpy(), w.dt_bias.double().numpy()
    lb = float(np.float32(w.lower_bound))
    worst = {}
    for n, (bb, a0, a1) in enumerate(seqs):
        for ci, c0 in enumerate(range(a0, a1, C)):
            c1 = min(c0 + C, a1)
            m = c1 - c0
            slot = first[n] + ci
            for h in range(H):
                idx = slot * H + h
                Qg, Mqk, Wm, U, Kbar, gn = _chunk_wy(q[bb, c0:c1, h], k[bb, c0:c1, h], v[bb, c0:c1, h],
                                                     g[bb, c0:c1, h], be[bb, c0:c1, h], A_log[h], dtb[h], lb)
                Wg = -_unfrag(frag("Wf", np.float16, C * K, idx), W_RC, (C, K))
                Qgg = _unfrag(frag("Qf", np.float16, C * K, idx), W_RC, (C, K))
                Kg = _unfrag(frag("Kf", np.float16, K * C, idx), K_RC, (K, C)).T
                Ag = _unfrag(frag("Af", np.float16, C * C, idx), A_RC, (C, C))
                Ug = _unfrag_u(frag("Uf", np.float16, C * V, idx))
                gng = frag("gn", np.float32, K, idx)
                for name, got, ref in (("W", Wg[:m], Wm), ("Qg", Qgg[:m], Qg), ("Kbar", Kg[:m], Kbar),
                                       ("U", Ug[:m], U), ("A_qk", np.tril(Ag[:m, :m]), Mqk)):
                    worst[name] = max(worst.get(name, 0.0), _close(got, ref, "%s seq %d chunk %d head %d" % (name, n, ci, h)))
                worst["gn"] = max(worst.get("gn", 0.0), _close(gng, gn, "gn", rel=1e-5))
                for name, got in (("W", Wg), ("Qg", Qgg), ("Kbar", Kg), ("U", Ug)):
                    assert not np.any(got[m:]), "%s rows past the end of a ragged chunk are not zero" % name
    say("case intermediates packed=%s: worst relative errors %s" % (packed, {k_: "%.1e" % v_ for k_, v_ in worst.items()}))
