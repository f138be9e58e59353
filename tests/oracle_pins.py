"""Pins of the fp64 oracle to things other than itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with what the mathematics fixes.  test_oracle_pins.py runs
them on the real oracle; test_oracle_mutants.py runs them on copies of the
oracle with planted mistakes and requires every mistake to be caught.

Kinds of pin:
  * independent routes: 40-digit brute force through explicit transition
    matrices (oracle/brute.py), and the chunk-parallel WY form in numpy
    (tests/chunked_model.py);
  * closed forms and hand-derivable values (T = 1, special gate values,
    decay by exactly 1/2 per token);
  * invariants: decay only when b = 0, delta-rule recall with orthogonal keys,
    overwrite with a repeated key, linearity in (v, S0), varlen packing ==
    separate calls, split run == full run, the contraction bound, head
    permutation.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import workloads as W

EPS = 1e-6


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _bf(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)


def _run(orc, w, **kw):
    return orc.fwd(w.q, w.k, w.v, w.g, w.beta, w.scale, w.A_log, w.dt_bias, w.lower_bound,
                   initial_state=kw.get("h0", w.initial_state), cu_seqlens=w.cu_seqlens)


def _hadamard(n):
    Hm = np.array([[1.0]])
    while Hm.shape[0] < n:
        Hm = np.block([[Hm, Hm], [Hm, -Hm]])
    return Hm


# ---------------------------------------------------------------- routes ----

def pin_brute_force(orc):
    """C oracle == 40-digit brute force through transition-matrix products."""
    from oracle import brute
    cases = [dict(K=2, T=5, lb=-5.0, init="fp32"), dict(K=4, T=9, lb=-1.0, init="fp32"),
             dict(K=8, T=12, lb=0.0, init=None), dict(K=4, T=7, lb=-3.0, init="fp32", g_mean=-2.0)]
    for i, c in enumerate(cases):
        w = W.make("bf", 1, c["T"], 2, 500 + i, K=c["K"], V=c["K"], lower_bound=c["lb"], init=c["init"],
                   g_mean=c.get("g_mean", 0.0))
        out, fin = _run(orc, w)
        h0 = None if w.initial_state is None else w.initial_state[0].double().numpy()
        bo, bfin = brute.run(_bits(w.q[0]), _bits(w.k[0]), _bits(w.v[0]), _bits(w.g[0]), _bits(w.beta[0]),
                             w.scale, w.A_log.numpy(), w.dt_bias.numpy(), w.lower_bound, h0)
        assert np.abs(out[0] - bo).max() <= 1e-12, ("brute out", i, np.abs(out[0] - bo).max())
        assert np.abs(fin[0] - bfin).max() <= 1e-12, ("brute state", i, np.abs(fin[0] - bfin).max())


def pin_chunked_form(orc):
    """C oracle == the chunk-parallel WY form, for several chunk sizes, ragged and packed."""
    from tests.chunked_model import chunked_forward
    w = W.make("ck", 1, 150, 2, 600, K=16, V=8, init="fp32", g_mean=-1.0)
    out, fin = _run(orc, w)
    for C in (1, 7, 64):
        co, cf = chunked_forward(w, C)
        assert np.abs(out - co).max() <= 1e-12, ("chunked out", C, np.abs(out - co).max())
        assert np.abs(fin - cf).max() <= 1e-11, ("chunked state", C, np.abs(fin - cf).max())
    wp = W.make("ckp", 1, 140, 2, 601, K=8, V=8, init="fp32", seqlens=[70, 1, 0, 69])
    out, fin = _run(orc, wp)
    co, cf = chunked_forward(wp, 16)
    assert np.abs(out - co).max() <= 1e-12 and np.abs(fin - cf).max() <= 1e-11, "chunked packed"


# ----------------------------------------------------------- closed forms ---

def pin_gate_values(orc):
    """Special values of a = max(lb, -exp(A_log) softplus(g + dt_bias))."""
    ln2 = math.log(2.0)
    assert abs(orc.softplus(0.0) - ln2) < 1e-15
    assert abs(orc.softplus(math.log(math.e - 1.0)) - 1.0) < 1e-15
    assert abs(orc.softplus(-40.0) - math.exp(-40.0)) < 1e-30
    assert abs(orc.softplus(40.0) - 40.0) < 1e-14
    for x in (-3.0, -0.5, 0.7, 5.0):  # softplus(x) - softplus(-x) = x
        assert abs(orc.softplus(x) - orc.softplus(-x) - x) < 1e-14
    assert abs(orc.gate(0.0, 0.0, 0.0, -5.0) + ln2) < 1e-15          # rate 1, step ln 2
    assert abs(orc.gate(0.25, 0.0, -0.25, -5.0) + ln2) < 1e-15       # dt_bias adds to g
    assert abs(orc.gate(math.log(math.e - 1.0), math.log(3.0), 0.0, -5.0) + 3.0) < 1e-14
    assert orc.gate(2.0, math.log(16.0), 0.0, -5.0) == -5.0           # clamped at the lower bound
    assert orc.gate(-3.0, 1.0, 0.0, 0.0) == 0.0                       # lb = 0 => no decay
    assert orc.gate(-math.inf, 0.0, 0.0, -5.0) == 0.0                 # g = -inf => no decay
    assert orc.gate(math.inf, 0.0, 0.0, -2.0) == -2.0                 # g = +inf => lower bound
    gs = np.linspace(-20, 20, 401)
    vals = np.array([orc.gate(x, 0.3, 0.1, -4.0) for x in gs])
    assert (vals <= 0).all() and (vals >= -4.0).all() and (np.diff(vals) <= 0).all()
    assert orc.sigmoid(0.0) == 0.5 and orc.sigmoid(math.inf) == 1.0 and orc.sigmoid(-math.inf) == 0.0


def pin_single_token(orc):
    """T = 1 from zero state: S1 = b khat v^T and o1 = scale b (khat . qhat) v, by hand:
    k = (3, 4), q = (1, 0), v = (2, -1), beta = 0 (b = 1/2), scale = 1/2."""
    w = W.make("t1", 1, 1, 1, 700, K=2, V=2, lower_bound=-5.0, init=None)
    w.k = _bf([[[[3.0, 4.0]]]]); w.q = _bf([[[[1.0, 0.0]]]]); w.v = _bf([[[[2.0, -1.0]]]])
    w.beta = _bf([[[0.0]]]); w.scale = 0.5
    out, fin = _run(orc, w)
    nk = math.sqrt(25.0 + EPS)
    kh = np.array([3.0, 4.0]) / nk
    qk = (3.0 / nk) / math.sqrt(1.0 + EPS)
    expect_o = 0.5 * 0.5 * qk * np.array([2.0, -1.0])
    expect_S = 0.5 * np.outer(kh, [2.0, -1.0])
    assert np.abs(out[0, 0, 0] - expect_o).max() < 1e-15, (out[0, 0, 0], expect_o)
    assert np.abs(fin[0, 0] - expect_S).max() < 1e-15


def pin_two_tokens(orc):
    """T = 2, no decay (lb = 0), b = 1, unit keys e1 then (e1+e2)/sqrt2, S0 = 0:
    S1 = e1 v1^T;  u2 = v2 - S1^T k2 = v2 - v1/sqrt2;  S2 = S1 + k2 u2^T;
    o2 = S2^T q2 with q2 = e2 -> v1 * 0 + u2 / sqrt2 (up to the L2-norm epsilon)."""
    w = W.make("t2", 1, 2, 1, 701, K=2, V=2, lower_bound=0.0, init=None)
    w.k = _bf([[[[1.0, 0.0]], [[1.0, 1.0]]]]); w.q = _bf([[[[1.0, 0.0]], [[0.0, 1.0]]]])
    w.v = _bf([[[[1.0, 2.0]], [[-3.0, 0.5]]]]); w.beta = _bf([[[math.inf], [math.inf]]]); w.scale = 1.0
    out, fin = _run(orc, w)
    r1 = 1.0 / math.sqrt(1.0 + EPS)
    r2 = 1.0 / math.sqrt(2.0 + EPS)
    k1 = np.array([r1, 0.0]); k2 = np.array([r2, r2])
    v1 = np.array([1.0, 2.0]); v2 = np.array([-3.0, 0.5])
    S1 = np.outer(k1, v1)
    u2 = v2 - S1.T @ k2
    S2 = S1 + np.outer(k2, u2)
    assert np.abs(out[0, 0, 0] - S1.T @ (k1 * 1.0)).max() < 1e-15
    assert np.abs(out[0, 1, 0] - S2.T @ np.array([0.0, r1])).max() < 1e-15
    assert np.abs(fin[0, 0] - S2).max() < 1e-15
    # and the recall property: S2^T k2 = v2 (both keys unit up to eps)
    assert np.abs(S2.T @ k2 - v2).max() < 1e-5


def pin_decay_only(orc):
    """b = 0 (beta = -inf): the state only decays.  With g = dt_bias = A_log = 0 each token
    halves it exactly; with A_log = ln 16 every channel is clamped to exp(lb)."""
    for A_val, lb, per in ((0.0, -5.0, 0.5), (math.log(16.0), -5.0, math.exp(-5.0)), (0.0, 0.0, 1.0)):
        w = W.make("dec", 1, 9, 2, 702, K=8, V=4, lower_bound=lb, init="fp32")
        w.beta = torch.full((1, 9, 2), -math.inf).to(torch.bfloat16)
        w.g = torch.zeros_like(w.g); w.dt_bias = torch.zeros_like(w.dt_bias)
        w.A_log = torch.full_like(w.A_log, A_val)
        out, fin = _run(orc, w)
        S0 = w.initial_state[0].double().numpy()
        assert np.abs(fin[0] - per ** 9 * S0).max() <= 1e-15 * max(1.0, np.abs(S0).max()), (A_val, lb)
        qn = w.q.double().numpy()[0]
        qn = qn / np.sqrt((qn ** 2).sum(-1, keepdims=True) + EPS)
        for t in range(9):
            expect = w.scale * np.einsum("hdj,hd->hj", per ** (t + 1) * S0, qn[t])
            assert np.abs(out[0, t] - expect).max() < 1e-14, (A_val, t)


# ------------------------------------------------------------- invariants ---

def pin_hadamard_recall(orc):
    """lb = 0, b = 1, keys = rows of a +-1 Hadamard matrix: after writing keys
    0..t, S^T khat_i = v_i for i <= t; with q = k every output reads back its
    value, and writing all K keys overwrites the initial state entirely."""
    K = 8
    Hm = _hadamard(K)
    w = W.make("had", 1, K, 2, 703, K=K, V=4, lower_bound=0.0, init="fp32")
    w.k = _bf(np.broadcast_to(Hm[None, :, None, :], (1, K, 2, K)).copy())
    w.q = w.k.clone()
    w.beta = torch.full((1, K, 2), math.inf).to(torch.bfloat16)
    out, fin = _run(orc, w)
    v = w.v.double().numpy()[0]
    # |khat|^2 = K / (K + eps): reading back is exact up to a relative eps / K
    assert np.abs(out[0] - w.scale * v).max() < 2e-6
    kh = Hm / math.sqrt(K + EPS)
    expect = np.einsum("td,thj->hdj", kh, v)  # state layout: S[d][j] = sum_t khat_t[d] v_t[j]
    assert np.abs(fin[0] - expect).max() < 1e-6
    for h in range(2):
        assert np.abs(fin[0, h].T @ kh.T - v[:, h].T).max() < 1e-6


def pin_overwrite(orc):
    """The same key written repeatedly with b = 1, no decay: the newest value wins."""
    w = W.make("ow", 1, 6, 1, 704, K=4, V=3, lower_bound=0.0, init="fp32")
    key = np.array([0.5, -1.0, 2.0, 0.25])
    w.k = _bf(np.broadcast_to(key, (1, 6, 1, 4)).copy()); w.q = w.k.clone()
    w.beta = torch.full((1, 6, 1), math.inf).to(torch.bfloat16)
    out, fin = _run(orc, w)
    kh = key / math.sqrt((key ** 2).sum() + EPS)
    v = w.v.double().numpy()[0, :, 0]
    for t in range(6):
        assert np.abs(out[0, t, 0] - w.scale * v[t]).max() < 1e-6
    assert np.abs(fin[0, 0].T @ kh - v[-1]).max() < 1e-6


def pin_linearity(orc):
    """For fixed q, k, g, beta the map (v, S0) -> (o, S_T) is linear (exactly
    representable inputs: quarter-integers)."""
    rng = np.random.default_rng(705)
    w1 = W.make("lin", 1, 20, 2, 705, K=8, V=6, init="fp32")
    v1 = rng.integers(-4, 5, size=w1.v.shape) / 4.0
    v2 = rng.integers(-4, 5, size=w1.v.shape) / 4.0
    s1 = torch.from_numpy(rng.integers(-4, 5, size=w1.initial_state.shape) / 8.0)
    s2 = torch.from_numpy(rng.integers(-4, 5, size=w1.initial_state.shape) / 8.0)
    res = []
    for v_, s_ in ((v1, s1), (v2, s2), (v1 + v2, s1 + s2)):
        w1.v = _bf(v_)
        res.append(_run(orc, w1, h0=s_))
    assert np.abs(res[0][0] + res[1][0] - res[2][0]).max() < 1e-13
    assert np.abs(res[0][1] + res[1][1] - res[2][1]).max() < 1e-13


def pin_varlen_separate(orc):
    """Packing sequences with cu_seqlens equals running them one by one (bitwise)."""
    lens = [5, 0, 17, 1, 9]
    w = W.make("pk", 1, sum(lens), 2, 706, K=8, V=4, init="fp32", seqlens=lens)
    out, fin = _run(orc, w)
    s = 0
    for n, L in enumerate(lens):
        ws = W.Workload("one", 1, L, 2, 8, 4, w.q[:, s:s + L], w.k[:, s:s + L], w.v[:, s:s + L],
                        w.g[:, s:s + L], w.beta[:, s:s + L], w.A_log, w.dt_bias, w.lower_bound, w.scale,
                        w.initial_state[n:n + 1], torch.float32, None, [L])
        o1, f1 = _run(orc, ws)
        assert np.array_equal(o1[0], out[0, s:s + L]) and np.array_equal(f1[0], fin[n]), n
        s += L


def pin_split_run(orc):
    """Running [0, t1) then [t1, T) from the first part's final state equals one run."""
    w = W.make("sp", 1, 23, 2, 707, K=8, V=4, init="fp32")
    out, fin = _run(orc, w)
    a = W.Workload("a", 1, 10, 2, 8, 4, w.q[:, :10], w.k[:, :10], w.v[:, :10], w.g[:, :10], w.beta[:, :10],
                   w.A_log, w.dt_bias, w.lower_bound, w.scale, w.initial_state, torch.float32, None, [10])
    oa, fa = _run(orc, a)
    b = W.Workload("b", 1, 13, 2, 8, 4, w.q[:, 10:], w.k[:, 10:], w.v[:, 10:], w.g[:, 10:], w.beta[:, 10:],
                   w.A_log, w.dt_bias, w.lower_bound, w.scale, None, torch.float32, None, [13])
    ob, fb = _run(orc, b, h0=fa)
    assert np.abs(np.concatenate([oa, ob], axis=1) - out).max() < 1e-14
    assert np.abs(fb - fin).max() < 1e-14


def pin_contraction(orc):
    """||S_t||_2 <= ||S_{t-1}||_2 + b_t ||khat_t|| ||v_t||, since each transition
    (I - b k k^T) Diag(exp(a)) has spectral norm <= 1."""
    w = W.make("ct", 1, 12, 1, 708, K=6, V=5, lower_bound=0.0, init="fp32", beta_std=3.0)
    S = w.initial_state
    kk = w.k.double().numpy()[0, :, 0]
    vv = w.v.double().numpy()[0, :, 0]
    bb = 1.0 / (1.0 + np.exp(-w.beta.double().numpy()[0, :, 0]))
    prev = np.linalg.norm(S[0, 0].double().numpy(), 2)
    for t in range(12):
        one = W.Workload("c", 1, 1, 1, 6, 5, w.q[:, t:t + 1], w.k[:, t:t + 1], w.v[:, t:t + 1],
                         w.g[:, t:t + 1], w.beta[:, t:t + 1], w.A_log, w.dt_bias, w.lower_bound, w.scale,
                         S, torch.float32, None, [1])
        _, f = _run(orc, one)
        cur = np.linalg.norm(f[0, 0], 2)
        kn = np.linalg.norm(kk[t]) / math.sqrt((kk[t] ** 2).sum() + EPS)
        assert cur <= prev + bb[t] * kn * np.linalg.norm(vv[t]) + 1e-12, t
        prev = cur
        S = torch.from_numpy(f)


def pin_head_permutation(orc):
    """Permuting heads together with A_log, dt_bias and S0 permutes the results."""
    w = W.make("hp", 1, 15, 3, 709, K=8, V=4, init="fp32")
    out, fin = _run(orc, w)
    p = [2, 0, 1]
    wp = w.head_slice(p)
    op, fp = _run(orc, wp)
    assert np.array_equal(op, out[:, :, p]) and np.array_equal(fp, fin[:, p])


def pin_golden(orc):
    """Stored 40-digit brute-force values (tests/golden/brute_small.json)."""
    import json
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "brute_small.json")
    with open(path) as f:
        gd = json.load(f)
    for case in gd["cases"]:
        sh = case["shape"]
        T, H, K, V = sh["T"], sh["H"], sh["K"], sh["V"]
        arr = lambda name, shape: np.array(case[name], dtype=np.uint16).reshape(shape)
        q, k, g = (arr(n, (1, T, H, K)) for n in ("q", "k", "g"))
        v = arr("v", (1, T, H, V))
        beta = arr("beta", (1, T, H))
        h0 = None if case["initial_state"] is None else np.array(case["initial_state"]).reshape(1, H, K, V)
        out, fin = orc.fwd(q, k, v, g, beta, case["scale"], np.array(case["A_log"], np.float32),
                           np.array(case["dt_bias"], np.float32), case["lower_bound"], initial_state=h0)
        eo = np.array([float(x) for x in case["out"]]).reshape(1, T, H, V)
        ef = np.array([float(x) for x in case["final_state"]]).reshape(1, H, K, V)
        assert np.abs(out - eo).max() <= 1e-12, ("golden out", case["name"])
        assert np.abs(fin - ef).max() <= 1e-12, ("golden state", case["name"])


ALL_PINS = [pin_brute_force, pin_chunked_form, pin_gate_values, pin_single_token, pin_two_tokens,
            pin_decay_only, pin_hadamard_recall, pin_overwrite, pin_linearity, pin_varlen_separate,
            pin_split_run, pin_contraction, pin_head_permutation, pin_golden]
