"""GPU parity of the single-token recurrent step (kda_decode, through the C ABI)
against the fp64 oracle, which runs the same token recurrence with T = 1 per
sequence (and over the whole sequence for prefill-then-decode)."""
import pytest
import torch

import gated_delta_rule_110_amd as kda
import workloads as W
from tests.parity import compare, run_oracle, say, to_np

pytestmark = pytest.mark.gpu


def _decode(w, initial, final, dev="cuda"):
    wd = w.to(dev)
    out, fin = kda.decode(wd.q, wd.k, wd.v, wd.g, wd.beta, w.scale, None, wd.A_log, wd.dt_bias,
                          w.lower_bound, initial, final)
    torch.cuda.synchronize()
    return out, fin


# (sequence, head) counts: up to 128 -> 4 column slices per head, up to 512 -> 2, above -> 1
@pytest.mark.parametrize("N,H,init,final", [(5, 6, "fp32", "fp32"), (3, 4, "bf16", "bf16"),
                                            (4, 2, None, "fp32"), (16, 16, "fp32", "bf16"),
                                            (64, 32, "fp32", "fp32")])
def test_decode_vs_oracle(N, H, init, final):
    w = W.make("decode", N, 1, H, 5000 + N * H, lower_bound=-4.0, init=init, final=final)
    say("case decode N=%d H=%d init=%s final=%s" % (N, H, init, final))
    h0 = None if w.initial_state is None else w.initial_state.to("cuda")
    ht = torch.empty((N, H, 128, 128), dtype=w.final_state_dtype, device="cuda")
    out, fin = _decode(w, h0, ht)
    ro, rf = run_oracle(w)
    compare(to_np(out), ro, to_np(fin), rf, w.final_state_dtype, "decode N=%d H=%d" % (N, H))


def test_decode_in_place_and_no_state_write():
    w = W.make("decode_ip", 6, 1, 3, 5101, init="fp32", final="fp32")
    say("case decode in place")
    h0 = w.initial_state.to("cuda")
    ref_out, ref_fin = _decode(w, h0, torch.empty_like(h0))
    ref_out, ref_fin = ref_out.clone(), ref_fin.clone()
    st = h0.clone()
    out, fin = _decode(w, st, st)
    assert fin.data_ptr() == st.data_ptr()
    assert torch.equal(out, ref_out) and torch.equal(st, ref_fin)
    # no final state: the output is still produced and the state is untouched
    keep = h0.clone()
    out2, fin2 = _decode(w, keep, None)
    assert fin2 is None and torch.equal(out2, ref_out) and torch.equal(keep, h0)


@pytest.mark.parametrize("state_dtype", [torch.float32, torch.bfloat16])
def test_prefill_then_decode(state_dtype):
    # prefill 200 tokens with kda_fwd, then three decode steps continuing the
    # state in place; compare with the oracle over all 203 tokens
    T0, steps, H = 200, 3, 4
    w = W.make("pd", 2, T0 + steps, H, 5202, lower_bound=-5.0, init="fp32", final="fp32")
    say("case prefill %d + decode %d, state %s" % (T0, steps, state_dtype))
    wd = w.to("cuda")
    st = torch.empty((2, H, 128, 128), dtype=state_dtype, device="cuda")
    h0 = wd.initial_state.to(state_dtype)
    pre = [t[:, :T0].contiguous() for t in (wd.q, wd.k, wd.v, wd.g, wd.beta)]
    out_pre, _ = kda.fwd(*pre, w.scale, None, wd.A_log, wd.dt_bias, w.lower_bound, h0, st)
    outs = [out_pre]
    for s in range(T0, T0 + steps):
        one = [t[:, s:s + 1].contiguous() for t in (wd.q, wd.k, wd.v, wd.g, wd.beta)]
        o, _ = kda.decode(*one, w.scale, None, wd.A_log, wd.dt_bias, w.lower_bound, st, st)
        outs.append(o)
    torch.cuda.synchronize()
    out = torch.cat(outs, dim=1)
    if state_dtype == torch.bfloat16:
        w.initial_state = w.initial_state.to(torch.bfloat16)  # the oracle sees the same rounded start
    ro, rf = run_oracle(w)
    compare(to_np(out), ro, to_np(st), rf, state_dtype, "prefill+decode %s" % state_dtype)


def test_decode_streamed_state_matches_cached():
    # 128 sequences x 32 heads of fp32 state is 256 MiB: the step streams the state past the
    # Infinity Cache (non-temporal loads and stores); the same step on a bf16 state of the same
    # shape (128 MiB) is cached.  Both must match the oracle; in place, the streamed step must
    # equal the out-of-place one bit for bit.
    N, H = 128, 32
    w = W.make("decode_stream", N, 1, H, 5301, lower_bound=-5.0, init="fp32", final="fp32")
    say("case decode streamed N=%d H=%d (fp32 state %d MiB)" % (N, H, N * H * 64 // 1024))
    h0 = w.initial_state.to("cuda")
    out, fin = _decode(w, h0, torch.empty_like(h0))
    ro, rf = run_oracle(w)
    compare(to_np(out), ro, to_np(fin), rf, torch.float32, "decode streamed")
    st = h0.clone()
    out2, _ = _decode(w, st, st)
    assert torch.equal(out2, out) and torch.equal(st, fin)
    wb = W.make("decode_stream", N, 1, H, 5301, lower_bound=-5.0, init="bf16", final="bf16")
    hb = wb.initial_state.to("cuda")
    outb, finb = _decode(wb, hb, torch.empty_like(hb))
    rob, rfb = run_oracle(wb)
    compare(to_np(outb), rob, to_np(finb), rfb, torch.bfloat16, "decode cached bf16")
