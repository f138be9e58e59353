"""Launches split into pieces (include/kda.h, "Launch size").

A batch too big for one launch of 2^30 work-items is enqueued as several
launches of the same kernel, each covering a range of chain groups, chunk rows
or decode units.  The descriptor's launch_piece cap makes small inputs take
that path.  Every (sequence, head) is computed by the same code either way, so
the results must be bit-identical to one launch, and within the usual
tolerances of the oracle.
"""
import pytest
import torch

import gated_delta_rule_110_amd as kda
import workloads as W
from tests.parity import compare, run_gpu, run_oracle, say, to_np

pytestmark = pytest.mark.gpu


def _same(a, b):
    return (a is None and b is None) or torch.equal(a, b)


def _check_fwd(w, pieces, label, chain_segments=0):
    ref_out, ref_fin = run_gpu(w, chain_segments=chain_segments)
    ro, rf = run_oracle(w)
    for p in pieces:
        say("case %s: launch_piece=%d" % (label, p))
        out, fin = run_gpu(w, chain_segments=chain_segments, launch_piece=p)
        assert _same(out, ref_out) and _same(fin, ref_fin), (label, p)
        compare(to_np(out), ro, to_np(fin), rf, w.final_state_dtype, "%s piece %d" % (label, p))


def test_packed_batch_in_pieces():
    # 11 sequences (two empty, ragged, chunk multiples) x 4 heads = 44 chains: the two-block
    # chain kernel in 6 groups of 8, and 22 chunk rows for the intra kernel
    lens = [0, 70, 1, 130, 64, 5, 0, 200, 33, 64, 129]
    w = W.make("pieces_packed", 1, sum(lens), 4, 6100, lower_bound=-4.0, init="fp32", final="fp32",
               seqlens=lens)
    _check_fwd(w, [1, 3, 1000000], "packed")


def test_fixed_batch_in_pieces():
    # 3 x 5 = 15 chains: the one-block chain kernel in 2 groups, 15 chunk rows
    w = W.make("pieces_fixed", 3, 300, 5, 6101, lower_bound=-5.0, init="bf16", final="bf16")
    _check_fwd(w, [1, 2], "fixed")


@pytest.mark.parametrize("H", [5, 9])
def test_split_chains_in_pieces(H):
    # 4 segments x H heads: 20 map chains in 3 groups (one-block passes), or 36 in 5 groups
    # (two-block passes), then the chains from the entering states
    w = W.make("pieces_split", 1, 64 * 13 + 7, H, 6102, lower_bound=-5.0, init="fp32", final="fp32")
    assert kda.chain_segments_for(w.B, w.T, w.H, 4) == 4
    _check_fwd(w, [1], "split H=%d" % H, chain_segments=4)


@pytest.mark.parametrize("init,final", [("fp32", "fp32"), ("bf16", "bf16")])
def test_decode_in_pieces(init, final):
    # 9 x 7 = 63 (sequence, head) units; a set piece size uses the one-slice kernel, so a piece
    # larger than the batch (one launch) is the reference for bit-identity
    N, H = 9, 7
    w = W.make("pieces_decode", N, 1, H, 6103, lower_bound=-4.0, init=init, final=final)
    wd = w.to("cuda")
    res = {}
    for p in (1000000, 4, 1):
        say("case decode N=%d H=%d %s/%s: launch_piece=%d" % (N, H, init, final, p))
        ht = torch.empty((N, H, 128, 128), dtype=w.final_state_dtype, device="cuda")
        out, fin = kda.decode(wd.q, wd.k, wd.v, wd.g, wd.beta, w.scale, None, wd.A_log, wd.dt_bias,
                              w.lower_bound, wd.initial_state, ht, launch_piece=p)
        torch.cuda.synchronize()
        res[p] = (out, fin)
    for p in (4, 1):
        assert torch.equal(res[p][0], res[1000000][0]) and torch.equal(res[p][1], res[1000000][1]), p
    ro, rf = run_oracle(w)
    compare(to_np(res[1][0]), ro, to_np(res[1][1]), rf, w.final_state_dtype, "decode pieces")
