"""kda_fwd_noalloc: the forward in the library's static scratch, for callers
that cannot allocate (graph capture, serving loops, harnesses without
hipMalloc).  Called through the C ABI, it must equal kda_fwd on the same
inputs bit for bit (the same kernels, another workspace) and meet the oracle's
tolerances, on two calls in a row with the second one smaller, so that the
second call runs over the scratch the first one left behind."""
import pytest
import torch

import gated_delta_rule_110_amd as kda
import workloads as W
from tests.parity import compare, run_oracle, say, to_np

pytestmark = pytest.mark.gpu


def _both(w):
    wd = w.to("cuda")
    outs = []
    for noalloc in (False, True):
        out = torch.full((w.B, w.T, w.H, w.V), float("nan"), dtype=torch.bfloat16, device="cuda")
        fin = None
        if w.final_state_dtype is not None:
            fin = torch.full((w.N, w.H, w.K, w.V), float("nan"), dtype=torch.float32, device="cuda")
            fin = fin.to(w.final_state_dtype)
        args = (wd.q, wd.k, wd.v, wd.g, wd.beta, w.scale, out, wd.A_log, wd.dt_bias, w.lower_bound,
                wd.initial_state, fin, wd.cu_seqlens)
        if noalloc:
            kda.fwd_noalloc(*args)
        else:
            kda.fwd(*args)
        torch.cuda.synchronize()
        outs.append((out, fin))
    return outs


def _check(w, label):
    say("case noalloc %s: B=%d T=%d H=%d N=%d (workspace %d of %d bytes)" %
        (label, w.B, w.T, w.H, w.N, kda.workspace_size(w.B, w.T, w.H, num_seqs=w.N), kda.noalloc_max_workspace()))
    (o1, f1), (o2, f2) = _both(w)
    assert torch.equal(o1, o2), label
    assert (f1 is None and f2 is None) or torch.equal(f1, f2), label
    ro, rf = run_oracle(w)
    compare(to_np(o2), ro, to_np(f2), rf, w.final_state_dtype, "noalloc " + label)


def test_noalloc_two_calls_second_smaller():
    # a packed batch with an empty and a one-token sequence (chunk table in the scratch) ...
    lens = [300, 0, 1, 200, 65]
    _check(W.make("noalloc_a", 1, sum(lens), 4, 9301, lower_bound=-4.0, init="fp32", final="fp32",
                  seqlens=lens), "packed")
    # ... then a smaller fixed-length batch over what the first call left behind
    _check(W.make("noalloc_b", 2, 130, 2, 9302, lower_bound=-5.0, init="bf16", final="bf16"), "fixed")


def test_noalloc_split_chains_fit():
    # the split-chain path also runs in the scratch (maps and entering states included)
    w = W.make("noalloc_split", 1, 64 * 40 + 9, 2, 9303, lower_bound=-5.0, init="fp32", final="fp32")
    say("case noalloc split chains")
    wd = w.to("cuda")
    out = torch.empty((1, w.T, w.H, 128), dtype=torch.bfloat16, device="cuda")
    fin = torch.empty((1, w.H, 128, 128), dtype=torch.float32, device="cuda")
    kda.fwd_noalloc(wd.q, wd.k, wd.v, wd.g, wd.beta, w.scale, out, wd.A_log, wd.dt_bias, w.lower_bound,
                    wd.initial_state, fin, None, chain_segments=4)
    ref_out = torch.empty_like(out)
    ref_fin = torch.empty_like(fin)
    kda.fwd(wd.q, wd.k, wd.v, wd.g, wd.beta, w.scale, ref_out, wd.A_log, wd.dt_bias, w.lower_bound,
            wd.initial_state, ref_fin, None, chain_segments=4)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(fin, ref_fin)


def test_noalloc_refuses_more_than_its_scratch():
    # 8192 tokens at 32 heads need about 290 MiB: refused on the host, nothing enqueued
    w = W.make("noalloc_big", 1, 8192, 32, 9304, init=None, final=None).to("cuda")
    out = torch.empty((1, 8192, 32, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kda.KdaArgumentError) as e:
        kda.fwd_noalloc(w.q, w.k, w.v, w.g, w.beta, w.scale, out, w.A_log, w.dt_bias, w.lower_bound)
    assert e.value.status == 9
