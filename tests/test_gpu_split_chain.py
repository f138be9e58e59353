"""GPU parity of split state chains (kda_desc_t::chain_segments) against the fp64 oracle.

A split chain computes every segment's affine state map on the GPU, composes
the maps in an fp32 scan and re-runs each segment from its entering state.
The result must meet the same tolerances as the unsplit path (bf16 outputs
max-abs 2e-2 and relative RMS 5e-3, fp32 states 1e-3, bf16 states 5e-3), and
stay close to the unsplit GPU result.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_110_amd as kda
import workloads as W
from tests.parity import compare, run_gpu, run_oracle, say, to_np

pytestmark = pytest.mark.gpu


def _check_split(w, segs, label, expect_segs=None):
    got = kda.chain_segments_for(w.B, w.T, w.H, segs)
    say("case %s: B=%d T=%d H=%d chain_segments=%d -> %d segments" % (label, w.B, w.T, w.H, segs, got))
    if expect_segs is not None:
        assert got == expect_segs
    out, fin = run_gpu(w, chain_segments=segs)
    ro, rf = run_oracle(w)
    res = compare(to_np(out), ro, to_np(fin), None if fin is None else rf, w.final_state_dtype, label)
    say("  vs oracle %s" % res)
    out1, fin1 = run_gpu(w, chain_segments=1)
    d = (out.float() - out1.float()).abs().max().item()
    say("  split vs unsplit: out max diff %.3e" % d)
    assert d <= 2e-2
    if fin is not None:
        rel = ((fin.float() - fin1.float()).norm() / fin1.float().norm()).item()
        say("  split vs unsplit: state rel %.3e" % rel)
        assert rel <= (5e-3 if w.final_state_dtype == torch.bfloat16 else 1e-3)
    return out, fin


@pytest.mark.parametrize("B,T,H,segs,init,final,expect", [
    (1, 64 * 40 + 17, 2, 4, "fp32", "fp32", 4),      # ragged last chunk in the last segment
    (2, 64 * 10 + 5, 3, 3, "bf16", "bf16", 3),       # two batch rows, bf16 states
    (1, 64 * 7, 1, 7, None, "fp32", 7),              # one chunk per segment, no initial state
    (1, 64 * 5 + 1, 2, 100, "fp32", "fp32", 6),      # more segments asked for than chunks
    (1, 64 * 9, 2, 4, "fp32", None, 3),              # no final state: the scan writes only entering states
    (2, 64 * 12 + 9, 5, 4, "fp32", "fp32", 4),       # 2 x 5 x 4 = 40 segment chains: the two-block chain pass
])
def test_split_matches_oracle(B, T, H, segs, init, final, expect):
    w = W.make("split", B, T, H, 5000 + T + segs, lower_bound=-5.0, init=init, final=final)
    _check_split(w, segs, "split%d T=%d" % (segs, T), expect)


def test_split_weak_decay_many_segments():
    # decays near 1: every segment's entering state carries most of the history, so the
    # composed maps (linear parts near the identity) must be accurate
    w = W.make("split-weak", 1, 4096, 2, 5101, lower_bound=-5.0, g_mean=-8.0, init="fp32", final="fp32")
    _check_split(w, 16, "split16 weak decay", 16)


def test_split_no_decay_lb0():
    w = W.make("split-lb0", 1, 2048, 2, 5102, lower_bound=0.0, init="fp32", final="fp32")
    _check_split(w, 8, "split8 lb=0", 8)


def test_split_in_place_state_and_poisoned_workspace():
    w = W.make("split-inplace", 1, 64 * 24 + 3, 3, 5103, init="fp32", final="fp32")
    ref_out, ref_fin = run_gpu(w, chain_segments=5)
    ref_out, ref_fin = ref_out.clone(), ref_fin.clone()
    say("case split in place + NaN-poisoned workspace")
    nbytes = kda.workspace_size(1, w.T, w.H, chain_segments=5)
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda").view(torch.uint8)
    state = w.initial_state.clone().to("cuda")
    wd = w.to("cuda")
    out = torch.full((1, w.T, w.H, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    kda.fwd(wd.q, wd.k, wd.v, wd.g, wd.beta, w.scale, out, wd.A_log, wd.dt_bias, w.lower_bound,
            state, state, None, workspace=ws, chain_segments=5)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    assert torch.equal(out, ref_out)
    assert torch.equal(state, ref_fin)


def test_split_long_few_heads_auto():
    # the bench workload for split chains at its full size: T = 131072, H = 4 (automatic split:
    # two rounds of 8 workgroups per segment and head over the 256 CUs)
    w = W.by_name("long_T131072_H4")
    segs = kda.chain_segments_for(w.B, w.T, w.H)
    assert segs == 16
    say("case %s: automatic split into %d segments" % (w.name, segs))
    out, fin = run_gpu(w)
    ro, rf = run_oracle(w)
    res = compare(to_np(out), ro, to_np(fin), rf, torch.float32, w.name)
    say("  vs oracle %s" % res)


def test_two_block_map_equals_one_block():
    # 8 segments x 8 heads = 64 (segment, head) chains: the map pass and the chain pass both
    # take two state blocks per workgroup; each 4-head half (32 chains) takes one block per
    # workgroup in both passes.  Heads are independent, so the results are equal bit for bit.
    w = W.make("map_x2", 1, 64 * 64 + 29, 8, 7801, lower_bound=-5.0, init="fp32", final="fp32")
    assert kda.chain_segments_for(w.B, w.T, w.H, 8) == 8
    say("case two-block map: T=%d H=8, 8 segments, against two 4-head halves" % w.T)
    out, fin = run_gpu(w, chain_segments=8)
    for lo in (0, 4):
        o, f = run_gpu(w.head_slice(range(lo, lo + 4)), chain_segments=8)
        assert torch.equal(out[:, :, lo:lo + 4], o) and torch.equal(fin[:, lo:lo + 4], f), lo
    ro, rf = run_oracle(w)
    compare(to_np(out), ro, to_np(fin), rf, torch.float32, "two-block map")
