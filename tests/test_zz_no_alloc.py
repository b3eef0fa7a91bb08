"""lh_forward_static (the forward that takes its workspace from the library's
static device scratch, for callers that cannot allocate) against lh_forward
through the C ABI: the same output bit for bit, on two calls in a row, the
second with a smaller input of another type and head size, then the first
shape again (the scratch keeps the previous call's contents)."""
import pytest
import torch

import sparse_long_context_lh_amd as lh
from parity import say
from synth_inputs import make_qkv

pytestmark = pytest.mark.gpu


def _one(N, H, d, L, p, k, dtype, seed):
    say("no-alloc forward: N=%d H=%d d=%d L=%d p=%d k=%d dtype=%s (forward workspace %.1f MiB of %.0f)"
        % (N, H, d, L, p, k, dtype, lh.forward_workspace_bytes(N, H, d, L, p, k, dtype) / 2 ** 20,
           lh.static_scratch_bytes() / 2 ** 20))
    q, kk, v = (x.cuda() for x in make_qkv(N, H, d, dtype, 8 if dtype == torch.bfloat16 else 0, seed))
    ref, _ = lh.forward(q, kk, v, L, p, k)
    got = lh.forward_static(q, kk, v, L, p, k)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    assert torch.all(torch.isfinite(got.float()))


def test_static_forward_matches_forward_twice():
    _one(16384, 2, 128, 3, 2, 300, torch.bfloat16, 31)    # 41 MiB of scratch
    _one(4096, 4, 64, 3, 2, 256, torch.float32, 32)       # smaller: the 4K fp32 workload, 14 MiB
    _one(16384, 2, 128, 3, 2, 300, torch.bfloat16, 33)    # larger again, over stale contents


def test_static_forward_rejects_a_shape_beyond_the_scratch():
    # the 64K workload's forward needs 1.3 GiB: refused before anything is queued
    N, H, d, L, p, k = 65536, 16, 128, 3, 2, 1536
    assert lh.forward_workspace_bytes(N, H, d, L, p, k, torch.bfloat16) > lh.static_scratch_bytes()
    q = torch.zeros(H, N, d, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lh.LighthouseError) as e:
        lh.forward_static(q, q, q, L, p, k)
    assert e.value.status == 2
