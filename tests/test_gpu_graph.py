"""kda_fwd under HIP graph capture: with a caller-owned workspace the forward
enqueues kernels only (no allocation, no memset), so it can be captured once
and replayed.  Every replay, with eager work and synchronisations between
replays, must reproduce the eager result bit for bit."""
import pytest
import torch

import gated_delta_rule_110_amd as kda
import workloads as W
from tests.parity import say

pytestmark = pytest.mark.gpu


def _buffers(w, chain_segments):
    ws = torch.empty(kda.workspace_size(w.B, w.T, w.H, num_seqs=w.N, chain_segments=chain_segments),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((w.B, w.T, w.H, w.V), dtype=torch.bfloat16, device="cuda")
    fin = torch.empty((w.N, w.H, w.K, w.V), dtype=w.final_state_dtype, device="cuda")
    return ws, out, fin


@pytest.mark.parametrize("case", ["fixed", "packed", "split", "split_wide"])
def test_graph_replays_match_eager(case):
    if case == "fixed":
        w, segs = W.make("graph-fixed", 2, 300, 3, 6001, init="fp32", final="fp32"), 0
    elif case == "packed":
        w, segs = W.make("graph-packed", 1, 260, 3, 6002, init="bf16", final="fp32", seqlens=[100, 0, 97, 63]), 0
    elif case == "split":
        w, segs = W.make("graph-split", 1, 64 * 12 + 9, 2, 6003, init="fp32", final="fp32"), 4
    else:  # 4 segments x 9 heads = 36 chains: two-block map and chain passes
        w, segs = W.make("graph-split-wide", 1, 64 * 12 + 9, 9, 6004, init="fp32", final="fp32"), 4
    say("case graph %s: B=%d T=%d H=%d N=%d chain_segments=%d" % (case, w.B, w.T, w.H, w.N, segs))
    wd = w.to("cuda")

    def call(ws, out, fin):
        kda.fwd(wd.q, wd.k, wd.v, wd.g, wd.beta, w.scale, out, wd.A_log, wd.dt_bias, w.lower_bound,
                wd.initial_state, fin, wd.cu_seqlens, workspace=ws, chain_segments=segs)

    ws_e, out_e, fin_e = _buffers(w, segs)
    call(ws_e, out_e, fin_e)
    torch.cuda.synchronize()

    ws, out, fin = _buffers(w, segs)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(ws, out, fin)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(ws, out, fin)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        fin.fill_(float("nan"))
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, out_e), (case, rep)
        assert torch.equal(fin, fin_e), (case, rep)
        say("  replay %d equals eager" % rep)


@pytest.mark.parametrize("N", [4, 128])   # 128 x 32 heads of fp32 state: the streamed decode kernel
def test_decode_graph_replays_match_eager(N):
    # three in-place decode steps captured once; each replay continues the state, and must equal
    # three more eager steps from the same state, bit for bit
    H, steps = (3, 3) if N == 4 else (32, 3)
    w = W.make("graph-decode", N, steps, H, 6100 + N, lower_bound=-5.0, init="fp32", final="fp32")
    say("case graph decode: N=%d H=%d, %d steps per replay" % (N, H, steps))
    wd = w.to("cuda")
    toks = [[t[:, s:s + 1].contiguous() for t in (wd.q, wd.k, wd.v, wd.g, wd.beta)] for s in range(steps)]
    outs_g = [torch.empty((N, 1, H, 128), dtype=torch.bfloat16, device="cuda") for _ in range(steps)]

    def run(st, outs):
        for s in range(steps):
            kda.decode(*toks[s], w.scale, outs[s], wd.A_log, wd.dt_bias, w.lower_bound, st, st)

    st_g = wd.initial_state.clone()
    graph = torch.cuda.CUDAGraph()
    warm = st_g.clone()
    run(warm, [torch.empty_like(o) for o in outs_g])  # warm-up outside the capture
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        run(st_g, outs_g)
    st_e = wd.initial_state.clone()
    st_g.copy_(wd.initial_state)
    for rep in range(3):
        outs_e = [torch.empty_like(o) for o in outs_g]
        run(st_e, outs_e)          # eager: the next three steps
        torch.cuda.synchronize()
        graph.replay()             # the same three steps from the graph's own state
        torch.cuda.synchronize()
        same = torch.equal(st_g, st_e) and all(torch.equal(a.view(torch.int16), b.view(torch.int16))
                                               for a, b in zip(outs_g, outs_e))
        say("  replay %d equal to eager: %s" % (rep, same))
        assert same
