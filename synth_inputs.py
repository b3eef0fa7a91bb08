"""Seeded synthetic inputs for the Lighthouse layer (no method arithmetic here).

Both the HIP path and the CPU oracle are fed from this module, and from nothing
else of each other. It only draws random numbers and lists the workload shapes.

Recipe (per workload): a generator seeded with ``seed`` draws, in this order,
  1. a per-token scale  s_n = exp(0.5 * z_n), z ~ N(0, 1)   (LogNormal(0, 0.5)),
  2. ``n_plant`` planted positions = the first n_plant of a random permutation
     of [0, N); the scale there is set to 4.0 (high-norm tokens),
  3. Q, then K, then V: for each head in order one [N, d] draw of N(0, 1),
     multiplied row-wise by s (the scale is per token: shared by heads and by
     Q, K and V),
  4. a cast to the workload dtype.
The upstream gradient dO is one N(0, 1) draw per head from a second generator
seeded ``seed + 1``.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    H: int
    d: int
    N: int
    L: int
    p: int
    k: int
    dtype: torch.dtype
    n_plant: int
    backward: bool


# The five workload shapes of the layer study (B = 1 folded into H).
WORKLOADS = [
    Workload("lh-fwd-4k-fp32", 4, 64, 4096, 3, 2, 256, torch.float32, 0, False),
    Workload("lh-fwd-64k", 16, 128, 65536, 3, 2, 1536, torch.bfloat16, 32, False),
    Workload("lh-fwd-128k", 16, 128, 131072, 3, 4, 1536, torch.bfloat16, 32, False),
    Workload("lh-fwdbwd-512k", 16, 128, 524288, 5, 4, 512, torch.bfloat16, 32, True),
    Workload("lh-fwdbwd-1m", 8, 128, 1048576, 6, 4, 1024, torch.bfloat16, 128, True),
]


# Dense causal attention over the whole sequence (L = 1: S = N, every token
# its own entry), the denominator of the layer's speedup at 512K tokens.
DENSE_WORKLOADS = [
    Workload("dense-fwdbwd-512k", 16, 128, 524288, 1, 2, 0, torch.bfloat16, 32, True),
]


# The (L, p, k) sweep at a fixed 512K tokens (H = 16, d = 128, bf16, 32
# planted tokens): p in {2, 4}, k from 512 to 6144, L = 3 or 5 where the
# pyramid allows it ((L-1) k <= 16384, k at most the top level's N/p^(L-1)
# entries). S runs from 10240 to 155648.
def _sweep():
    out = []
    for p in (2, 4):
        for L in (3, 5):
            for k in (512, 1536, 3072, 6144):
                if (L - 1) * k > 16384 or k > 524288 // p ** (L - 1):
                    continue
                out.append(Workload("sweep-512k-L%d-p%d-k%d" % (L, p, k), 16, 128, 524288, L, p, k,
                                    torch.bfloat16, 32, True))
    return out


SWEEP_WORKLOADS = _sweep()


def by_name(name: str) -> Workload:
    for w in WORKLOADS + DENSE_WORKLOADS + SWEEP_WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(name)


def make_qkv(N: int, H: int, d: int, dtype=torch.bfloat16, n_plant: int = 0,
             seed: int = 0, device: str = "cpu"):
    """Q, K, V as [H, N, d] tensors of ``dtype`` on ``device``.

    device="cpu" draws from torch's CPU generator; device="cuda" draws the same
    recipe from the device generator (a different stream of numbers, same
    distribution), which is far faster at million-token sizes.
    """
    g = torch.Generator(device=device).manual_seed(seed)
    scale = torch.exp(0.5 * torch.randn(N, generator=g, device=device, dtype=torch.float32))
    if n_plant:
        pos = torch.randperm(N, generator=g, device=device)[:n_plant]
        scale[pos] = 4.0
    out = []
    for _ in range(3):
        t = torch.empty(H, N, d, dtype=dtype, device=device)
        for h in range(H):
            z = torch.randn(N, d, generator=g, device=device, dtype=torch.float32)
            t[h] = (z * scale[:, None]).to(dtype)
        out.append(t)
    return tuple(out)


def make_dout(N: int, H: int, d: int, dtype=torch.bfloat16, seed: int = 1, device: str = "cpu"):
    """Upstream gradient dO as an [H, N, d] tensor: N(0, 1) per element."""
    g = torch.Generator(device=device).manual_seed(seed)
    t = torch.empty(H, N, d, dtype=dtype, device=device)
    for h in range(H):
        t[h] = torch.randn(N, d, generator=g, device=device, dtype=torch.float32).to(dtype)
    return t


def make_workload(w: Workload, seed: int = 0, device: str = "cpu", N: int | None = None, H: int | None = None):
    """Inputs of a workload (optionally with N or H overridden for small cases)."""
    n = w.N if N is None else N
    h = w.H if H is None else H
    q, k, v = make_qkv(n, h, w.d, w.dtype, min(w.n_plant, n), seed, device)
    return q, k, v


def make_layer_inputs(N: int, d_model: int, H: int, d: int, dtype=torch.bfloat16, n_plant: int = 0, seed: int = 0,
                      device: str = "cpu"):
    """The input x [N, d_model] and projection weights W [d_model, 3 H d] of
    the layer with its projections: x as the Q/K/V recipe above (per-token
    LogNormal(0, 0.5) scale, n_plant tokens at scale 4), W ~ N(0, 1/d_model)
    so the projected rows have about unit variance; W from seed + 2."""
    g = torch.Generator(device=device).manual_seed(seed)
    scale = torch.exp(0.5 * torch.randn(N, generator=g, device=device, dtype=torch.float32))
    if n_plant:
        pos = torch.randperm(N, generator=g, device=device)[:n_plant]
        scale[pos] = 4.0
    x = (torch.randn(N, d_model, generator=g, device=device, dtype=torch.float32) * scale[:, None]).to(dtype)
    gw = torch.Generator(device=device).manual_seed(seed + 2)
    w = (torch.randn(d_model, 3 * H * d, generator=gw, device=device, dtype=torch.float32)
         / d_model ** 0.5).to(dtype)
    return x, w
