"""GPU edge cases of the in-kernel activations and of the delta rule itself.

The q/k L2 norm, the beta sigmoid and the gate all run inside the kernels
("作为 FLA 后端的用法", zuobiaodaohang.com FlashKDA page; the gate's parameters
and the [-5, 0] lower bound, "Debajo del capó: CUTLASS en Hopper",
7minutos.es), so their extreme inputs are exercised here against the oracle:

* beta = -inf makes b = 0: no token writes, and the state only decays,
  S_T = Diag(exp(sum_t a_t)) S_0.  The per-channel log-decay sum is then read
  back from the GPU's final state, log(S_T[d, :] / S_0[d, :]), and compared
  channel by channel with the sum of the oracle's gate values: this pins the
  kernel's gate function itself, not only its effect on the outputs.  Gates
  near 0 (g about -15, where softplus(g) is about 3e-7) over a long sequence,
  g = +-inf, and g + dt_bias far above the point where exp overflows in fp32
  (with A_log so small that the lower bound does not hide the result).
* beta = +inf makes b = 1 (a full delta-rule overwrite) with decays active.
* All-zero q or k rows inside a chunk: a zero key writes nothing and a zero
  query reads zero.
"""
import dataclasses

import numpy as np
import pytest
import torch

import gated_delta_rule_110_amd as kda
import oracle
import workloads as W
from tests.parity import compare, run_gpu, run_oracle, say, to_np

pytestmark = pytest.mark.gpu


def _oracle_gate_sums(w):
    """sum over tokens of the oracle's per-channel log-decay, [N, H, K] (fixed-length batches)."""
    g = w.g.float().numpy().astype(np.float64)
    A = w.A_log.numpy().astype(np.float64)
    dtb = w.dt_bias.numpy().astype(np.float64)
    lb = w.lower_bound
    B, T, H, K = g.shape
    sums = np.zeros((B, H, K))
    for b in range(B):
        for h in range(H):
            for d in range(K):
                sums[b, h, d] = sum(oracle.gate(float(x), float(A[h]), float(dtb[h, d]), lb) for x in g[b, :, h, d])
    return sums


def _recovered_gate_sums(fin, h0):
    """log of the per-row ratio S_T / S_0 (least squares over the row's V entries)."""
    num = np.einsum("nhkv,nhkv->nhk", fin, h0)
    den = np.einsum("nhkv,nhkv->nhk", h0, h0)
    return np.log(num / den)


def _decay_only(w):
    return dataclasses.replace(w, beta=torch.full(w.beta.shape, float("-inf")).to(torch.bfloat16))


def _check_decay_only(w, label):
    assert w.initial_state is not None and w.final_state_dtype == torch.float32
    say("case decay-only %s: B=%d T=%d H=%d lb=%g" % (label, w.B, w.T, w.H, w.lower_bound))
    out, fin = run_gpu(w)
    ro, rf = run_oracle(w)
    compare(to_np(out), ro, to_np(fin), rf, torch.float32, "decay-only " + label)
    got = _recovered_gate_sums(to_np(fin), w.initial_state.double().numpy())
    want = _oracle_gate_sums(w)
    err = np.abs(got - want)
    tol = 1e-5 + 1e-4 * np.abs(want)
    i = np.unravel_index(np.argmax(err / tol), err.shape)
    say("  sum_t a_t per channel: range [%.4g, %.4g], worst |err| %.3e at %s (tol %.3e)" %
        (want.min(), want.max(), err[i], i, tol[i]))
    assert np.isfinite(got).all(), label
    assert (err <= tol).all(), (label, i, got[i], want[i])


def test_decay_only_moderate_gate():
    # g ~ N(-6, 1): a about -0.04 per token; 200 tokens over four chunks, the last ragged
    _check_decay_only(_decay_only(W.make("b0", 1, 200, 3, 8101, lower_bound=-5.0, g_mean=-6.0,
                                         init="fp32", final="fp32")), "g~N(-6,1)")


def test_decay_only_tiny_gate_long():
    # g ~ N(-15, 1): softplus(g) about 3e-7, where log(1 + e^x) in fp32 loses the low bits of
    # e^x (and returns 0 below x = -16.6); 4096 tokens accumulate sum a of about -0.02
    _check_decay_only(_decay_only(W.make("b0tiny", 1, 4096, 2, 8102, lower_bound=-5.0, g_mean=-15.0,
                                         init="fp32", final="fp32")), "g~N(-15,1)")


def _extreme_gates(w, A_log):
    """g = +inf, -inf, 95, 100 (x = g + dt_bias past fp32 exp overflow) and -100 on a fixed
    pattern of (token, channel), normal values elsewhere; per-head A_log as given."""
    g = w.g.float().clone()
    B, T, H, K = g.shape
    t = torch.arange(T)[:, None, None]
    d = torch.arange(K)[None, None, :]
    sel = (t * 3 + d) % 11
    vals = {0: float("inf"), 1: float("-inf"), 2: 95.0, 3: 100.0, 4: -100.0}
    for key, val in vals.items():
        g = torch.where((sel == key)[None].expand(B, T, H, K), torch.full_like(g, val), g)
    return dataclasses.replace(w, g=g.to(torch.bfloat16), A_log=torch.tensor(A_log, dtype=torch.float32))


@pytest.mark.parametrize("lb", [-0.5, -5.0])
def test_gate_extremes(lb):
    # A_log = -12 makes exp(A_log) = 6e-6, so a = -6e-6 * softplus(100) = -6e-4 stays above the
    # lower bound: an exp overflow inside softplus would show as the clamp instead
    A_log = [-12.0, -6.0, 0.0, 2.7]
    w = _extreme_gates(W.make("gext", 1, 70, 4, 8103, lower_bound=lb, g_mean=-1.0, init="fp32",
                              final="fp32"), A_log)
    gv = w.g.float()
    assert torch.isinf(gv).any() and (gv == 100.0).any() and (gv == -100.0).any()
    say("case extreme gates lb=%g: forward" % lb)
    out, fin = run_gpu(w)
    ro, rf = run_oracle(w)
    compare(to_np(out), ro, to_np(fin), rf, torch.float32, "extreme gates lb=%g" % lb)
    if lb == -0.5:  # sum a >= -35 over 70 tokens: the decayed state stays well inside fp32
        _check_decay_only(_decay_only(w), "extreme gates lb=%g" % lb)


def test_decode_gate_extremes():
    # one decode step with b = 0: the state's rows scale by exp(a), so a itself is read back
    N, H = 4, 4
    w = _extreme_gates(W.make("gdec", N, 1, H, 8104, lower_bound=-0.5, g_mean=-1.0, init="fp32",
                              final="fp32"), [-12.0, -6.0, 0.0, 2.7])
    # every batch row gets the same token pattern: vary it over rows instead
    g = w.g.float()
    for n in range(N):
        g[n] = torch.roll(g[n], shifts=n, dims=-1)
    w = _decay_only(dataclasses.replace(w, g=g.to(torch.bfloat16)))
    say("case decode extreme gates")
    wd = w.to("cuda")
    out, fin = kda.decode(wd.q, wd.k, wd.v, wd.g, wd.beta, w.scale, None, wd.A_log, wd.dt_bias,
                          w.lower_bound, wd.initial_state, torch.empty_like(wd.initial_state))
    torch.cuda.synchronize()
    ro, rf = run_oracle(w)
    compare(to_np(out), ro, to_np(fin), rf, torch.float32, "decode extreme gates")
    got = _recovered_gate_sums(to_np(fin), w.initial_state.double().numpy())
    want = _oracle_gate_sums(w)
    err = np.abs(got - want)
    assert (err <= 1e-5 + 1e-4 * np.abs(want)).all(), float(err.max())


def test_beta_pos_inf_with_decay():
    # b = 1 on every token: each write fully replaces the key's component; decays down to -5
    w = W.make("b1", 2, 300, 3, 8105, lower_bound=-5.0, init="fp32", final="fp32")
    w = dataclasses.replace(w, beta=torch.full(w.beta.shape, float("inf")).to(torch.bfloat16))
    say("case beta=+inf lb=-5")
    out, fin = run_gpu(w)
    ro, rf = run_oracle(w)
    compare(to_np(out), ro, to_np(fin), rf, torch.float32, "beta=+inf lb=-5")


def test_zero_query_and_key_rows():
    # zero rows at chunk edges, a whole 16-row block of one chunk, and q-only / k-only rows
    w = W.make("zrows", 1, 200, 3, 8106, lower_bound=-5.0, init="fp32", final="fp32")
    q, k = w.q.clone(), w.k.clone()
    both = [0, 15, 16, 17, 31, 63, 64, 127, 128, 199] + list(range(80, 96))
    q[:, both] = 0
    k[:, both] = 0
    q[:, [5, 70, 150]] = 0
    k[:, [6, 71, 151]] = 0
    w = dataclasses.replace(w, q=q, k=k)
    say("case zero q/k rows")
    out, fin = run_gpu(w)
    ro, rf = run_oracle(w)
    compare(to_np(out), ro, to_np(fin), rf, torch.float32, "zero q/k rows")
    o = to_np(out)
    zq = both + [5, 70, 150]
    assert np.abs(o[:, zq]).max() == 0.0  # a zero query reads exactly zero
