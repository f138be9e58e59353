"""GPU parity: libkda (through the C ABI) against the fp64 oracle.

Every case draws seeded synthetic inputs (workloads.py), runs kda_fwd on the
GPU and the plain token recurrence on the CPU, and compares element by
element: bf16 outputs within max-abs 2e-2 and relative RMS 5e-3, fp32 final
states within relative 1e-3, bf16 final states within 5e-3.
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from tests.parity import compare, run_gpu, run_oracle, say, to_np

pytestmark = pytest.mark.gpu


def _check(w, label, heads=None):
    say("case %s: B=%d T=%d H=%d N=%d lb=%g" % (label, w.B, w.T, w.H, w.N, w.lower_bound))
    out, fin = run_gpu(w)
    if heads is not None:
        # heads are independent: compare a sample of them against the oracle
        ws = w.head_slice(heads)
        ro, rf = run_oracle(ws)
        og = to_np(out)[:, :, list(heads)]
        fg = None if fin is None else to_np(fin)[:, list(heads)]
    else:
        ro, rf = run_oracle(w)
        og, fg = to_np(out), to_np(fin)
    return compare(og, ro, fg, None if fin is None else rf, w.final_state_dtype, label)


@pytest.mark.parametrize("idx", [0, 1, 2, 3])
def test_config_full(idx):
    w = W.config(idx)
    _check(w, W.CONFIG_NAMES[idx])


@pytest.mark.parametrize("name", W.PAGES_NAMES)
def test_pages_workloads(name):
    # the pages' benchmark shapes: T = 8192, H = 96 / 64, fixed length and 8 x 1024 packed
    w = W.pages_workload(name)
    _check(w, name)


def test_config4_all_heads():
    # T = 131072, H = 32: one GPU call, then the oracle on 16 heads at a time (heads are
    # independent), so that its fp64 output stays at about 2 GB of host memory per batch
    w = W.config(4)
    say("case %s: B=%d T=%d H=%d (oracle in two batches of 16 heads)" % (W.CONFIG_NAMES[4], w.B, w.T, w.H))
    out, fin = run_gpu(w)
    for h0 in range(0, w.H, 16):
        heads = list(range(h0, min(w.H, h0 + 16)))
        ws = w.head_slice(heads)
        ro, rf = run_oracle(ws)
        og = out[:, :, heads[0]:heads[-1] + 1].float().cpu().double().numpy()
        fg = to_np(fin[:, heads[0]:heads[-1] + 1])
        compare(og, ro, fg, rf, w.final_state_dtype, "%s heads %d-%d" % (W.CONFIG_NAMES[4], heads[0], heads[-1]))
        del ro, rf, og


@pytest.mark.parametrize("lens", [[1], [37], [63], [64], [65], [127], [200, 1, 64, 65, 37, 300]])
def test_ragged_varlen(lens):
    w = W.make("ragged", 1, sum(lens), 3, 2000 + sum(lens), lower_bound=-4.0, init="fp32",
               final="fp32", seqlens=lens)
    _check(w, "ragged%s" % lens)


def test_many_short_sequences():
    # more sequences than one workgroup of the chunk-table scan covers (1024), with empty ones:
    # the scan's carry across blocks, and thousands of (sequence, head) chains
    rng = np.random.Generator(np.random.PCG64(4242))
    lens = [int(x) for x in rng.integers(0, 41, size=1100)]
    lens[0] = lens[500] = lens[1024] = lens[-1] = 0
    w = W.make("many", 1, sum(lens), 2, 4243, lower_bound=-4.0, init="fp32", final="fp32", seqlens=lens)
    _check(w, "many%d" % len(lens))


@pytest.mark.parametrize("T", [1, 63, 65, 200])
def test_fixed_ragged_tail(T):
    w = W.make("tail", 2, T, 3, 3000 + T, init="bf16", final="fp32")
    _check(w, "tail T=%d" % T)


def test_weak_decay_state_path():
    # g ~ N(-8, 1): decays near 1, the state carries information across every chunk
    w = W.make("weak", 1, 4096, 4, 4001, lower_bound=-5.0, g_mean=-8.0, init="fp32", final="fp32")
    _check(w, "weak-decay")


def test_no_decay_lb0():
    w = W.make("nodecay", 2, 1024, 4, 4002, lower_bound=0.0, init="fp32", final="fp32")
    _check(w, "lb=0")


def test_no_initial_bf16_final():
    w = W.make("bf16fin", 1, 777, 4, 4003, init=None, final="bf16")
    _check(w, "init=None final=bf16")


def test_empty_sequences_and_T0():
    lens = [0, 70, 0, 5, 0]
    w = W.make("empty", 1, sum(lens), 2, 4004, init="fp32", final="fp32", seqlens=lens)
    _check(w, "empty-seqs")
    # T = 0 packed: final state = initial state exactly
    w0 = W.make("T0", 1, 0, 2, 4005, init="fp32", final="fp32", seqlens=[0, 0])
    say("case T=0")
    out, fin = run_gpu(w0)
    assert out.numel() == 0
    assert torch.equal(fin.cpu(), w0.initial_state)


def test_hadamard_recall_state_layout():
    # lb = 0 (no decay), beta = +inf (b = 1), keys = rows of a +-1 Hadamard
    # matrix: after writing keys 0..n-1, S^T khat_i = v_i, and with q = k every
    # output reads back its own value: o_t = scale * v_t.
    H, T, K = 2, 128, 128
    w = W.make("hadamard", 1, T, H, 4006, lower_bound=0.0, init="fp32", final="fp32")
    Hm = np.array([[1.0]])
    while Hm.shape[0] < K:
        Hm = np.block([[Hm, Hm], [Hm, -Hm]])
    keys = torch.from_numpy(Hm[:T].astype(np.float32)).to(torch.bfloat16)
    w.k = keys[None, :, None, :].expand(1, T, H, K).contiguous()
    w.q = w.k.clone()
    w.beta = torch.full((1, T, H), float("inf")).to(torch.bfloat16)
    say("case hadamard-recall")
    out, fin = run_gpu(w)
    o = to_np(out)[0]
    v = w.v.double().numpy()[0]
    err = np.abs(o - w.scale * v).max()
    say("  recall max err %.3e" % err)
    assert err <= 5e-3
    # all 128 keys written: the initial state is fully overwritten, S = sum_i khat_i v_i^T
    kh = Hm[:T] / math.sqrt(K + 1e-6)
    expect = np.einsum("td,thj->hdj", kh, v)
    f = to_np(fin)[0]
    rel = np.linalg.norm(f - expect) / np.linalg.norm(expect)
    say("  state rel %.3e" % rel)
    assert rel <= 1e-3
    ro, rf = run_oracle(w)
    compare(to_np(out), ro, to_np(fin), rf, torch.float32, "hadamard vs oracle")


def test_varlen_equals_separate_calls_bitwise():
    lens = [100, 64, 1, 250, 37]
    w = W.make("pack", 1, sum(lens), 3, 4007, init="fp32", final="fp32", seqlens=lens)
    say("case varlen == separate calls")
    out, fin = run_gpu(w)
    start = 0
    for n, L in enumerate(lens):
        ws = W.Workload("one", 1, L, w.H, w.K, w.V, w.q[:, start:start + L].contiguous(),
                        w.k[:, start:start + L].contiguous(), w.v[:, start:start + L].contiguous(),
                        w.g[:, start:start + L].contiguous(), w.beta[:, start:start + L].contiguous(),
                        w.A_log, w.dt_bias, w.lower_bound, w.scale,
                        w.initial_state[n:n + 1].contiguous(), torch.float32, None, [L])
        o1, f1 = run_gpu(ws)
        assert torch.equal(o1.cpu(), out[:, start:start + L].cpu()), n
        assert torch.equal(f1.cpu(), fin[n:n + 1].cpu()), n
        start += L


def test_split_run_equals_full_run():
    T, t1 = 700, 301  # split point not on a chunk boundary
    w = W.make("split", 1, T, 3, 4008, g_mean=-4.0, init="fp32", final="fp32")
    say("case split == full")
    out, fin = run_gpu(w)

    def part(a, b, h0):
        return W.Workload("p", 1, b - a, w.H, w.K, w.V, w.q[:, a:b].contiguous(), w.k[:, a:b].contiguous(),
                          w.v[:, a:b].contiguous(), w.g[:, a:b].contiguous(), w.beta[:, a:b].contiguous(),
                          w.A_log, w.dt_bias, w.lower_bound, w.scale, h0, torch.float32, None, [b - a])
    o1, f1 = run_gpu(part(0, t1, w.initial_state))
    o2, f2 = run_gpu(part(t1, T, f1.cpu()))
    ro, rf = run_oracle(w)
    compare(to_np(torch.cat([o1, o2], dim=1)), ro, to_np(f2), rf, torch.float32, "split run vs oracle")
    d = (torch.cat([o1, o2], dim=1).float() - out.float()).abs().max().item()
    say("  split vs full max diff %.3e" % d)
    assert d <= 2e-2


def test_deterministic_and_no_uninitialised_reads():
    w = W.make("det", 1, 1000, 4, 4009, init="fp32", final="fp32", seqlens=[300, 700])
    say("case determinism + NaN-poisoned buffers")
    import gated_delta_rule_110_amd as kda
    nbytes = kda.workspace_size(1, 1000, 4, num_seqs=2)
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda").view(torch.uint8)
    out = torch.full((1, 1000, 4, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    fin = torch.full((2, 4, 128, 128), float("nan"), dtype=torch.float32, device="cuda")
    o1, f1 = run_gpu(w, workspace=ws, out=out, final=fin)
    o1, f1 = o1.clone(), f1.clone()
    assert torch.isfinite(o1.float()).all() and torch.isfinite(f1).all()
    o2, f2 = run_gpu(w)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


def test_abi_errors_on_device():
    import gated_delta_rule_110_amd as kda
    w = W.make("err", 1, 64, 2, 4010, init=None, final=None).to("cuda")
    with pytest.raises(kda.KdaError) as e:
        kda.fwd(w.q, w.k, w.v, w.g, w.beta, w.scale, None, w.A_log, w.dt_bias, -6.0)
    assert e.value.status == 4
    assert isinstance(e.value, ValueError) and isinstance(e.value, kda.KdaArgumentError)
    with pytest.raises(kda.KdaError) as e:
        kda.fwd(w.q, w.k, w.v, w.g, w.beta, w.scale, None, w.A_log, w.dt_bias, 0.5)
    assert e.value.status == 4
