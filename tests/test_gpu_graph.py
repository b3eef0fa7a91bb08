"""The layer inside a captured HIP graph: the library allocates, copies and
clears nothing and never synchronises, so a forward + backward captured once
replays to the eager result, bit for bit (the path is deterministic)."""
import pytest
import torch

import sparse_long_context_lh_amd as lh
from parity import say
from synth_inputs import make_dout, make_qkv

pytestmark = pytest.mark.gpu


def test_graph_replay_matches_eager():
    N, H, d, L, p, k = 16384, 2, 128, 3, 4, 64
    say("case graph: N=%d H=%d d=%d L=%d p=%d k=%d" % (N, H, d, L, p, k))
    q, kk, v = (x.cuda() for x in make_qkv(N, H, d, torch.bfloat16, 8, 21))
    dout = make_dout(N, H, d, torch.bfloat16, 22).cuda()
    ws = lh.alloc_workspace(N, H, d, L, p, k, torch.bfloat16)
    out = torch.empty_like(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    res = (out, dq, dk, dv)

    def step():
        lh.forward(q, kk, v, L, p, k, ws=ws, out=out)
        lh.backward(dout, L, p, k, ws, dq, dk, dv)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in res]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # a warm-up on the capture stream's kind of stream
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in res:  # eager work between replays
            t.zero_()
        ws[: ws.numel() // 2].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(("out", "dq", "dk", "dv"), res, ref):
            assert torch.equal(t, r), "replay %d: %s differs from the eager result" % (rep, name)
    say("  graph: 3 replays equal the eager result")
