"""Calls on distinct workspaces may run at the same time: two forward + backward
passes of different shapes, queued on two streams at once, give bit for bit
what each gives alone (the kernels share no memory but their arguments)."""
import pytest
import torch

import sparse_long_context_lh_amd as lh
from parity import say
from synth_inputs import make_dout, make_qkv

pytestmark = pytest.mark.gpu


class _Job:
    def __init__(self, N, H, d, L, p, k, seed):
        self.shape = (L, p, k)
        self.q, self.k, self.v = (x.cuda() for x in make_qkv(N, H, d, torch.bfloat16, 8, seed))
        self.dout = make_dout(N, H, d, torch.bfloat16, seed + 1).cuda()
        self.ws = lh.alloc_workspace(N, H, d, L, p, k, torch.bfloat16)
        self.res = tuple(torch.empty_like(self.q) for _ in range(4))  # out, dq, dk, dv

    def run(self, stream=None):
        L, p, k = self.shape
        out, dq, dk, dv = self.res
        lh.forward(self.q, self.k, self.v, L, p, k, ws=self.ws, out=out, stream=stream)
        lh.backward(self.dout, L, p, k, self.ws, dq, dk, dv, stream=stream)


def test_two_streams_match_sequential():
    a = _Job(16384, 2, 128, 3, 4, 64, seed=31)
    b = _Job(32768, 3, 64, 4, 2, 200, seed=33)
    say("case streams: two jobs of shapes %s and %s" % ((16384, 2, 128, 3, 4, 64), (32768, 3, 64, 4, 2, 200)))
    a.run()
    b.run()
    torch.cuda.synchronize()
    ref_a = [t.clone() for t in a.res]
    ref_b = [t.clone() for t in b.res]
    for t in a.res + b.res:
        t.zero_()
    torch.cuda.synchronize()

    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
    for _ in range(3):  # several rounds, so launches of the two jobs interleave
        a.run(s1)
        b.run(s2)
    torch.cuda.synchronize()
    for got, want in zip(a.res + b.res, ref_a + ref_b):
        assert torch.equal(got, want)
