"""The intra kernel writes its intermediates with the non-temporal hint once
they reach 128 MiB (about 72.5 KiB per 64-token chunk and head).  The hint
changes where the lines are cached, never their values: heads are independent,
so a forward over 32 heads (148 MB of intermediates, streamed) must equal its
two 16-head halves (74 MB each, cached) bit for bit, and match the oracle."""
import pytest
import torch

import gated_delta_rule_110_amd as kda
import workloads as W
from tests.parity import compare, run_gpu, run_oracle, say, to_np

pytestmark = pytest.mark.gpu

STREAM_BYTES = 128 << 20


def test_streamed_equals_cached_halves():
    w = W.make("stream", 1, 4096, 32, 7701, lower_bound=-5.0, init="fp32", final="fp32")
    per_head = kda.workspace_size(1, w.T, 2) - kda.workspace_size(1, w.T, 1)
    assert per_head * 32 >= STREAM_BYTES > per_head * 16  # the full call streams, the halves do not
    say("case stream stores: T=4096 H=32 against two halves of 16 heads")
    out, fin = run_gpu(w)
    for lo in (0, 16):
        half = w.head_slice(range(lo, lo + 16))
        o, f = run_gpu(half)
        assert torch.equal(out[:, :, lo:lo + 16], o) and torch.equal(fin[:, lo:lo + 16], f), lo
    ro, rf = run_oracle(w)
    compare(to_np(out), ro, to_np(fin), rf, w.final_state_dtype, "stream T=4096 H=32")
