"""Pins of the oracle's gradient (kda_oracle_bwd.c), all on the CPU.

The gradient is the vector-Jacobian product of the forward recurrence: for
loss gradients (d_out, d_final) it returns the derivative of
L = <d_out, out> + <d_final, final_state> with respect to every input.  It is
pinned to things other than itself:

* central finite differences of the forward oracle, entry by entry, on tiny
  inputs (K, V <= 8) with an initial state, varlen sequences (one empty), both
  clamped and unclamped gate channels, and more than one 64-token checkpoint
  block (the reverse pass recomputes states from those checkpoints);
* the identity <VJP(u), w> = <u, JVP(w)>, with the JVP taken by torch's
  forward-mode differentiation of a plain fp64 torch recurrence (which is
  itself checked against the forward oracle first), at a moderate size;
* closed forms: with beta = -inf nothing is written and the state only decays,
  so every gradient is a sum of decayed products; a single token from a zero
  state gives o = scale b (qh . kh) v;
* the fp64-input forward agrees with the bf16-input forward oracle on the same
  values;
* planted mistakes in the gradient's C source (a dropped term, a wrong sign or
  index, a wrong checkpoint) each fail one of the pins above.
"""
import math
import os
import re

import numpy as np
import pytest
import torch

import oracle

EPS = oracle.EPS


def _inputs(B, T, H, K, V, seed, lb=-3.0, cu=None, init=True, g_shift=0.0):
    """Seeded fp64 inputs.  The gate inputs are spread so that some channels sit
    on the clamp (z << lb) and others well inside (|z - lb| >= 0.05), keeping
    finite differences away from the clamp's kink."""
    rng = np.random.default_rng(seed)
    N = B if cu is None else len(cu) - 1
    x = {
        "q": rng.standard_normal((B, T, H, K)),
        "k": rng.standard_normal((B, T, H, K)),
        "v": rng.standard_normal((B, T, H, V)),
        "g": rng.standard_normal((B, T, H, K)) * 2.0 + g_shift,
        "beta": rng.standard_normal((B, T, H)),
        "A_log": rng.uniform(-1.0, 0.5, H),
        "dt_bias": rng.standard_normal((H, K)) * 0.5,
        "initial_state": rng.standard_normal((N, H, K, V)) if init else None,
    }
    # push gate inputs away from the kink: z = -e^A softplus(g + dt) vs lb
    for _ in range(50):
        z = -np.exp(x["A_log"])[None, None, :, None] * np.logaddexp(0.0, x["g"] + x["dt_bias"][None, None])
        near = np.abs(z - lb) < 0.05
        if not near.any():
            break
        x["g"][near] -= 0.3
    d_out = rng.standard_normal((B, T, H, V))
    d_final = rng.standard_normal((N, H, K, V))
    return x, d_out, d_final, lb, 0.7, cu


def _loss(orc, x, d_out, d_final, lb, scale, cu):
    out, fin = orc.fwd_f64(x["q"], x["k"], x["v"], x["g"], x["beta"], scale, x["A_log"], x["dt_bias"], lb,
                           initial_state=x["initial_state"], cu_seqlens=cu)
    return float((out * d_out).sum() + (fin * d_final).sum())


def _grads(orc, x, d_out, d_final, lb, scale, cu):
    return orc.bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], scale, x["A_log"], x["dt_bias"], lb, d_out,
                   d_final=d_final, initial_state=x["initial_state"], cu_seqlens=cu)


GRAD_OF = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "A_log": "dA_log",
           "dt_bias": "ddt_bias", "initial_state": "d_initial"}


def _fd_check(orc, case, step=1e-6, rtol=1e-6, names=None):
    """Compare every gradient entry with a central difference of the loss.  Returns
    the worst |analytic - fd| / (1 + |fd|) and raises nothing (callers assert)."""
    x, d_out, d_final, lb, scale, cu = case
    gr = _grads(orc, x, d_out, d_final, lb, scale, cu)
    worst = 0.0
    for name in names or GRAD_OF:
        if x[name] is None:
            continue
        arr = x[name]
        flat = arr.reshape(-1)
        ana = gr[GRAD_OF[name]].reshape(-1)
        for i in range(flat.size):
            keep = flat[i]
            flat[i] = keep + step
            lp = _loss(orc, x, d_out, d_final, lb, scale, cu)
            flat[i] = keep - step
            lm = _loss(orc, x, d_out, d_final, lb, scale, cu)
            flat[i] = keep
            fd = (lp - lm) / (2 * step)
            worst = max(worst, abs(ana[i] - fd) / (1.0 + abs(fd)))
    return worst


CASES = {
    "dense": dict(B=2, T=5, H=2, K=4, V=4, seed=11),
    "k_ne_v": dict(B=1, T=6, H=2, K=5, V=3, seed=12),
    "varlen": dict(B=1, T=9, H=2, K=3, V=2, seed=13, cu=[0, 4, 4, 9]),
    "no_decay": dict(B=1, T=5, H=1, K=4, V=4, seed=14, lb=0.0),
    "all_clamped": dict(B=1, T=5, H=1, K=4, V=4, seed=15, lb=-0.01, g_shift=3.0),
}


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


@pytest.mark.parametrize("name", sorted(CASES))
def test_gradient_matches_central_differences(orc, name):
    c = dict(CASES[name])
    case = _inputs(c.pop("B"), c.pop("T"), c.pop("H"), c.pop("K"), c.pop("V"), **c)
    assert _fd_check(orc, case) < 1e-6


def test_gradient_across_checkpoint_blocks(orc):
    # 150 tokens: three checkpoint blocks (64, 64, 22) in the reverse pass; plus a varlen
    # split whose second sequence starts mid-block
    case = _inputs(1, 150, 1, 3, 2, seed=16, cu=[0, 70, 150])
    assert _fd_check(orc, case, names=["k", "g", "beta", "initial_state", "A_log", "dt_bias"]) < 1e-6


def test_clamped_channels_pass_no_gradient(orc):
    # every channel on the clamp: the gate is a constant lb, so g, dt_bias and A_log get nothing
    c = dict(CASES["all_clamped"])
    x, d_out, d_final, lb, scale, cu = _inputs(c.pop("B"), c.pop("T"), c.pop("H"), c.pop("K"), c.pop("V"), **c)
    z = -np.exp(x["A_log"])[None, None, :, None] * np.logaddexp(0.0, x["g"] + x["dt_bias"][None, None])
    assert (z < lb).all()
    gr = _grads(orc, x, d_out, d_final, lb, scale, cu)
    assert not gr["dg"].any() and not gr["dA_log"].any() and not gr["ddt_bias"].any()


# --- the JVP identity, against torch forward-mode differentiation ----------------------------


def _torch_forward(q, k, v, g, beta, A_log, dt_bias, S0, scale, lb, cu):
    """Plain fp64 torch recurrence, differentiated by torch.func.jvp only."""
    B, T, H, K = q.shape
    seqs = [(b, 0, T) for b in range(B)] if cu is None else [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]
    outs = torch.zeros(B, T, H, v.shape[-1], dtype=torch.float64)
    fins = []
    for n, (b, r0, r1) in enumerate(seqs):
        per_head = []
        for h in range(H):
            S = S0[n, h]
            for t in range(r0, r1):
                qh = q[b, t, h] / torch.sqrt((q[b, t, h] ** 2).sum() + EPS)
                kh = k[b, t, h] / torch.sqrt((k[b, t, h] ** 2).sum() + EPS)
                bt = torch.sigmoid(beta[b, t, h])
                a = torch.clamp(-torch.exp(A_log[h]) * torch.nn.functional.softplus(g[b, t, h] + dt_bias[h]), min=lb)
                S = torch.exp(a)[:, None] * S
                u = bt * (v[b, t, h] - S.T @ kh)
                S = S + torch.outer(kh, u)
                outs = outs.index_put((torch.tensor(b), torch.tensor(t), torch.tensor(h)), scale * (S.T @ qh))
            per_head.append(S)
        fins.append(torch.stack(per_head))
    return outs, torch.stack(fins)


def test_vjp_equals_jvp_transpose(orc):
    B, T, H, K, V = 1, 150, 2, 8, 8
    cu = [0, 23, 150]
    x, d_out, d_final, lb, scale, _ = _inputs(B, T, H, K, V, seed=17, cu=cu)
    names = ["q", "k", "v", "g", "beta", "A_log", "dt_bias", "initial_state"]
    prim = tuple(torch.from_numpy(x[n].copy()) for n in names)
    rng = np.random.default_rng(18)
    tang = tuple(torch.from_numpy(rng.standard_normal(p.shape)) for p in prim)
    fn = lambda *a: _torch_forward(*a, scale, lb, cu)
    (o_t, f_t), (do_t, df_t) = torch.func.jvp(fn, prim, tang)
    # the torch recurrence is the oracle's forward (pinned elsewhere)
    o_ref, f_ref = orc.fwd_f64(x["q"], x["k"], x["v"], x["g"], x["beta"], scale, x["A_log"], x["dt_bias"], lb,
                               initial_state=x["initial_state"], cu_seqlens=cu)
    assert np.abs(o_t.numpy() - o_ref).max() < 1e-12 and np.abs(f_t.numpy() - f_ref).max() < 1e-12
    gr = _grads(orc, x, d_out, d_final, lb, scale, cu)
    lhs = sum(float((gr[GRAD_OF[n]] * t.numpy()).sum()) for n, t in zip(names, tang))
    rhs = float((d_out * do_t.numpy()).sum() + (d_final * df_t.numpy()).sum())
    assert abs(lhs - rhs) <= 1e-10 * (abs(rhs) + 1.0), (lhs, rhs)
    # and input by input, so that one wrong gradient cannot hide behind another
    for n, t in zip(names, tang):
        only = tuple(tt if nn == n else torch.zeros_like(tt) for nn, tt in zip(names, tang))
        (_, _), (do1, df1) = torch.func.jvp(fn, prim, only)
        r1 = float((d_out * do1.numpy()).sum() + (d_final * df1.numpy()).sum())
        l1 = float((gr[GRAD_OF[n]] * t.numpy()).sum())
        assert abs(l1 - r1) <= 1e-10 * (abs(r1) + 1.0), (n, l1, r1)


# --- closed forms -----------------------------------------------------------------------------


def _nrm(x):
    r = 1.0 / np.sqrt((x * x).sum(-1, keepdims=True) + EPS)
    return x * r, r


def test_no_write_closed_form(orc):
    """beta = -inf: b = 0, S_t = Diag(exp(A_t)) S_0 with A_t the running sum of the
    log-decays, o_t = scale S_t^T qh_t.  Then, per channel d,
      dL/da_s[d] = sum_{t>=s} scale qh_t[d] e^{A_t[d]} (S_0 do_t)[d] + e^{A_T[d]} (S_0 * dF)[d,:].sum()
    and nothing reaches k, v or beta."""
    B, T, H, K, V = 1, 7, 1, 4, 3
    x, d_out, d_final, lb, scale, cu = _inputs(B, T, H, K, V, seed=19)
    x["beta"][:] = -math.inf
    gr = _grads(orc, x, d_out, d_final, lb, scale, cu)
    assert not gr["dk"].any() and not gr["dv"].any() and not gr["dbeta"].any()
    S0 = x["initial_state"][0, 0]
    qh, rq = _nrm(x["q"][0, :, 0])
    z = -np.exp(x["A_log"][0]) * np.logaddexp(0.0, x["g"][0, :, 0] + x["dt_bias"][0])
    a = np.maximum(z, lb)
    At = np.cumsum(a, 0)  # [T, K]
    do = d_out[0, :, 0]
    S0do = do @ S0.T  # [T, K]: (S_0 do_t)[d]
    term = scale * qh * np.exp(At) * S0do  # per (t, d)
    da = np.cumsum(term[::-1], 0)[::-1] + np.exp(At[-1]) * (S0 * d_final[0, 0]).sum(1)
    mask = z > lb
    dz = np.where(mask, da, 0.0)
    sig = 1.0 / (1.0 + np.exp(-(x["g"][0, :, 0] + x["dt_bias"][0])))
    dg = -np.exp(x["A_log"][0]) * sig * dz
    np.testing.assert_allclose(gr["dg"][0, :, 0], dg, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(gr["ddt_bias"][0], dg.sum(0), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(gr["dA_log"][0], (z * dz).sum(), rtol=1e-12, atol=1e-13)
    dqh = scale * np.exp(At) * S0do
    dq = rq * dqh - rq ** 3 * (x["q"][0, :, 0] * dqh).sum(-1, keepdims=True) * x["q"][0, :, 0]
    np.testing.assert_allclose(gr["dq"][0, :, 0], dq, rtol=1e-12, atol=1e-13)
    dS0 = np.exp(At[-1])[:, None] * d_final[0, 0] + (scale * qh * np.exp(At)).T @ do
    np.testing.assert_allclose(gr["d_initial"][0, 0], dS0, rtol=1e-12, atol=1e-13)


def test_single_token_closed_form(orc):
    """One token from a zero state: S = b kh v^T, o = scale b (qh . kh) v."""
    K, V = 6, 5
    x, d_out, d_final, lb, scale, cu = _inputs(1, 1, 1, K, V, seed=20, init=False)
    gr = _grads(orc, x, d_out, d_final, lb, scale, cu)
    q, k, v, do, dF = x["q"][0, 0, 0], x["k"][0, 0, 0], x["v"][0, 0, 0], d_out[0, 0, 0], d_final[0, 0]
    qh, rq = _nrm(q)
    kh, rk = _nrm(k)
    b = 1.0 / (1.0 + math.exp(-x["beta"][0, 0, 0]))
    c = qh @ kh
    np.testing.assert_allclose(gr["dv"][0, 0, 0], scale * b * c * do + b * (kh @ dF), rtol=1e-12)
    db = scale * c * (v @ do) + kh @ dF @ v
    np.testing.assert_allclose(gr["dbeta"][0, 0, 0], db * b * (1 - b), rtol=1e-12)
    dqh = scale * b * (v @ do) * kh
    dkh = scale * b * (v @ do) * qh + b * (dF @ v)
    np.testing.assert_allclose(gr["dq"][0, 0, 0], rq * dqh - rq ** 3 * (q @ dqh) * q, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(gr["dk"][0, 0, 0], rk * dkh - rk ** 3 * (k @ dkh) * k, rtol=1e-11, atol=1e-13)
    assert not gr["dg"].any() and not gr["dA_log"].any() and not gr["ddt_bias"].any()
    np.testing.assert_allclose(gr["d_initial"][0, 0], np.zeros((K, V)) + gr["d_initial"][0, 0])  # shape


def test_zero_loss_gradient_gives_zero(orc):
    x, d_out, d_final, lb, scale, cu = _inputs(2, 9, 2, 4, 4, seed=21)
    gr = _grads(orc, x, np.zeros_like(d_out), np.zeros_like(d_final), lb, scale, cu)
    assert all(not v.any() for v in gr.values())


def test_f64_forward_agrees_with_bf16_forward(orc):
    # the same values through both entry points: bf16-exact inputs, fp32 parameters
    rng = np.random.default_rng(22)
    B, T, H, K, V = 2, 70, 2, 16, 8
    bf = lambda shape: torch.from_numpy(rng.standard_normal(shape)).to(torch.bfloat16)
    q, k, g = bf((B, T, H, K)), bf((B, T, H, K)), bf((B, T, H, K))
    v, beta = bf((B, T, H, V)), bf((B, T, H))
    A_log = torch.from_numpy(rng.uniform(-1, 0.5, H)).float()
    dtb = torch.from_numpy(rng.standard_normal((H, K))).float()
    S0 = torch.from_numpy(rng.standard_normal((B, H, K, V)))
    scale, lb = float(np.float32(K ** -0.5)), float(np.float32(-4.0))
    o1, f1 = orc.fwd(q, k, v, g, beta, scale, A_log, dtb, lb, initial_state=S0)
    o2, f2 = orc.fwd_f64(q.double(), k.double(), v.double(), g.double(), beta.double(), scale, A_log.double(),
                         dtb.double(), lb, initial_state=S0)
    assert np.abs(o1 - o2).max() <= 1e-12 * max(1.0, np.abs(o1).max())
    assert np.abs(f1 - f2).max() <= 1e-12 * max(1.0, np.abs(f1).max())


def test_bad_arguments_are_rejected(orc):
    x, d_out, d_final, lb, scale, _ = _inputs(1, 6, 1, 2, 2, seed=23)
    with pytest.raises(ValueError):
        orc.bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], scale, x["A_log"], x["dt_bias"], lb, d_out,
                cu_seqlens=[0, 4, 3])
    with pytest.raises(ValueError):
        orc.bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], scale, x["A_log"], x["dt_bias"], lb, d_out,
                cu_seqlens=[0, 4, 5])


# --- planted mistakes -------------------------------------------------------------------------

MUTANTS = [
    ("drop the norm's projection", "- rq3 * qd * q[qk + d]", ""),
    ("wrong sign of the S' read", "dkh[d] -= t.b * s;", "dkh[d] += t.b * s;"),
    ("no decay on the carried gradient", "G[d * V + j] = dec[d] * gs;", "G[d * V + j] = gs;"),
    ("decay gradient from the undecayed state", "da += gs * Sp[d * V + j];", "da += gs * Sprev[d * V + j];"),
    ("dA_log without the gate value", "dz_sum += z[d] * tmp[d];", "dz_sum += tmp[d];"),
    ("sigmoid derivative dropped", "db * t.b * (1.0 - t.b)", "db * t.b"),
    ("dv without b", "dv[vo + (size_t)j] = t.b * du[j];", "dv[vo + (size_t)j] = du[j];"),
    ("gradient through the clamp", "if (z[d] > lower_bound) {", "if (1) {"),
    ("output gradient on the old state", "s += Snow[d * V + j] * dov[j];", "s += Sp[d * V + j] * dov[j];"),
    ("wrong checkpoint state", "? blk + (size_t)(row - r0 - 1) * KV", "? blk + (size_t)(row - r0) * KV"),
    ("r read against the transposed state", "for (int64_t d = 0; d < K; ++d) s += Sp[d * V + j] * kh[d];",
     "for (int64_t d = 0; d < K; ++d) s += Sp[j * V + d] * kh[d];"),
    ("shared gradients from one sequence", "for (int64_t n = 0; n < N; ++n) s += pA[n * H + h];",
     "for (int64_t n = 0; n < 1; ++n) s += pA[n * H + h];"),
]


@pytest.mark.parametrize("label,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistakes_are_caught(tmp_path, label, old, new):
    src = oracle.source_bwd()
    assert src.count(old) == 1, label
    lib = oracle.compile_variant(oracle.source(), str(tmp_path / "mut.so"), bwd_text=src.replace(old, new))
    mut = oracle.Oracle(lib)
    caught = False
    for case in (_inputs(1, 9, 2, 3, 2, seed=13, cu=[0, 4, 4, 9]),
                 _inputs(2, 5, 2, 4, 4, seed=11),
                 _inputs(1, 70, 1, 2, 2, seed=24)):
        if _fd_check(mut, case) > 1e-4:
            caught = True
            break
    assert caught, label
