"""Lighthouse Attention layer for one MI355X (gfx950): HIP kernels behind a C ABI.

The layer pools Q, K and V into an L-level average pyramid with factor p,
scores tokens by the l2 norms of their query and key rows (max-pooled up the
pyramid), keeps a stratified top-k per level, gathers the chosen entries into
one causally ordered sub-sequence of length S = N/p^(L-1) + (L-1)*p*k, runs
dense causal attention over it and scatters every output back over its
causal-safe shifted range. ``forward`` / ``backward`` call liblh.so; see
include/lh.h for the ABI.
"""
from .binding import (LighthouseError, alloc_workspace, backward, check_shape, ds_tile_budget, forward,  # noqa: F401
                      forward_nograd, forward_static, forward_workspace_bytes, layer_backward, layer_forward,
                      layer_qkv, layer_workspace_bytes, lib, padded_subseq_len, region, selection, selftest_sqrt, set_ds_tile_budget,
                      stage_names, static_scratch_bytes, subseq_len, workspace_bytes)
