"""The C ABI without a GPU: the library loads, exports every function the
header declares, and validates arguments before queueing any HIP work."""
import json
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lh.h")


@pytest.fixture(scope="module")
def L():
    from sparse_long_context_lh_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from sparse_long_context_lh_amd.build import build_library
        build_library()
    return binding.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lh_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = _declared_functions()
    assert "lh_forward" in names and "lh_backward" in names
    for name in names:
        assert hasattr(L, name), name


def test_subseq_len_golden(L):
    with open(os.path.join(ROOT, "tests", "golden", "subseq_lengths.json")) as f:
        for c in json.load(f)["cases"]:
            assert L.lh_subseq_len(c["N"], c["L"], c["p"], c["k"]) == c["S"]
            assert L.lh_padded_subseq_len(c["N"], c["L"], c["p"], c["k"]) % 256 == 0


@pytest.mark.parametrize("args,code", [
    ((4096, 4, 64, 3, 2, 256, 1), 0),
    ((4098, 4, 64, 3, 2, 256, 0), 1),      # N not a multiple of p^(L-1)
    ((4096, 4, 64, 3, 2, 1025, 0), 1),     # k > N / p^(L-1)
    ((4096, 4, 64, 3, 2, -1, 0), 1),       # negative k
    ((4096, 4, 96, 3, 2, 16, 0), 3),       # d outside {64, 128}
    ((4096, 4, 60, 3, 2, 16, 0), 1),       # d not a multiple of 16
    ((2 * 7168, 1, 128, 2, 2, 4, 0), 1),   # level of 7168 entries: not a multiple of the stratum
    ((4096, 4, 64, 3, 3, 16, 0), 3),       # p not a power of two
    ((4096, 4, 64, 3, 1, 16, 0), 1),       # p < 2 with L > 1
    ((4096, 4, 64, 0, 2, 16, 0), 1),       # L < 1
    ((4096, 4, 64, 9, 2, 1, 0), 3),        # L > 8
    ((4096, 0, 64, 3, 2, 16, 0), 1),       # H < 1
    ((0, 4, 64, 1, 0, 0, 0), 1),           # N = 0: nothing to attend
    ((-64, 4, 64, 3, 2, 1, 0), 1),         # N < 0
    ((4096, 65536, 64, 3, 2, 16, 0), 3),   # H > 65535
    ((4096, 4, 64, 3, 2, 16, 7), 1),       # unknown dtype
    ((4096, 4, 64, 1, 0, 0, 0), 0),        # L = 1: dense causal attention, p unused
])
def test_shape_validation(L, args, code):
    assert L.lh_check_shape(*args) == code
    ws = L.lh_workspace_bytes(*args)
    assert (ws > 0) == (code == 0)


def test_forward_rejects_before_any_device_call(L):
    shape = (4096, 4, 64, 3, 2, 256, 0)
    need = L.lh_workspace_bytes(*shape)
    need_fwd = L.lh_forward_workspace_bytes(*shape)
    fake = 1 << 40  # never dereferenced: validation fails first
    # bad shape
    assert L.lh_forward(fake, fake, fake, 4098, 4, 64, 3, 2, 256, 0, fake, fake, need, None) == 1
    # null input pointer
    assert L.lh_forward(None, fake, fake, *shape, fake, fake, need, None) == 1
    # misaligned output pointer
    assert L.lh_forward(fake, fake, fake, *shape, fake + 2, fake, need, None) == 1
    # workspace too small, null, misaligned
    assert L.lh_forward(fake, fake, fake, *shape, fake, fake, need_fwd - 1, None) == 2
    assert L.lh_forward(fake, fake, fake, *shape, fake, None, need, None) == 2
    assert L.lh_forward(fake, fake, fake, *shape, fake, fake + 16, need, None) == 2
    # backward: same checks
    assert L.lh_backward(fake, *shape, fake, fake, fake, fake, need - 1, None) == 2
    assert L.lh_backward(None, *shape, fake, fake, fake, fake, need, None) == 1
    assert L.lh_forward_timed(fake, fake, fake, *shape, fake, fake, need, None, None) == 1


def test_workspace_regions_disjoint(L):
    import ctypes
    from sparse_long_context_lh_amd.binding import REGIONS
    shape = (65536, 16, 128, 3, 2, 1536, 0)
    total = L.lh_workspace_bytes(*shape)
    spans = []
    for r in range(len(REGIONS)):
        off, nb = ctypes.c_size_t(), ctypes.c_size_t()
        assert L.lh_region_info(*shape, r, ctypes.byref(off), ctypes.byref(nb)) == 0
        assert off.value % 256 == 0
        spans.append((off.value, off.value + nb.value))
    spans.sort()
    for a, b in zip(spans, spans[1:]):
        assert a[1] <= b[0]
    assert spans[-1][1] <= total
    assert L.lh_region_info(*shape, len(REGIONS), ctypes.byref(off), ctypes.byref(nb)) == 1


def test_unused_fp16_copies_take_no_space(L):
    # no kernel reads Q hi transposed; with bf16 inputs the lo parts of Q and
    # K exist only as the library's internal e4m3 tiles (Q) or not at all (K)
    from sparse_long_context_lh_amd.binding import REGIONS
    for dt, lo_bytes in ((0, 0), (1, 2 * 4 * 2048 * 64)):
        shape = (4096, 4, 64, 3, 2, 256, dt)
        assert _region(L, shape, REGIONS.index("qhi_t"))[1] == 0
        assert _region(L, shape, REGIONS.index("khi_t"))[1] == 2 * 4 * 2048 * 64
        assert _region(L, shape, REGIONS.index("qlo"))[1] == lo_bytes
        assert _region(L, shape, REGIONS.index("klo"))[1] == lo_bytes


def test_stage_names(L):
    from sparse_long_context_lh_amd import binding
    assert binding.stage_names(False) == ["front", "topk", "index", "gather", "attn_fwd", "scatter"]
    assert binding.stage_names(True) == ["scatter_bwd", "bwd_prep", "attn_bwd_dkdv", "attn_bwd_dq", "pool_bwd"]


def test_size_helpers_do_not_depend_on_head_size(L):
    # S and S_pad need N, L, p and k only: N = 2^24 at L = 1 is a valid
    # d = 64 shape (S_pad * d = 2^30) even though d = 128 would exceed 2^30
    assert L.lh_subseq_len(1 << 24, 1, 2, 0) == 1 << 24
    assert L.lh_padded_subseq_len(1 << 24, 1, 2, 0) == 1 << 24
    assert L.lh_check_shape(1 << 24, 1, 64, 1, 2, 0, 0) == 0
    assert L.lh_check_shape(1 << 24, 1, 128, 1, 2, 0, 0) == 3
    assert L.lh_subseq_len(4098, 3, 2, 1) == -1


def test_huge_workspace_is_unsupported_not_wrapped(L):
    # 65535 heads of 2^24 tokens would need petabytes: reported, never wrapped
    assert L.lh_workspace_bytes(1 << 24, 65535, 64, 1, 2, 0, 0) == 0
    assert L.lh_check_shape(1 << 24, 65535, 64, 1, 2, 0, 0) == 3


def _region(L, shape, r):
    import ctypes
    off, nb = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.lh_region_info(*shape, r, ctypes.byref(off), ctypes.byref(nb)) == 0
    return off.value, nb.value


def test_forward_workspace_is_a_prefix(L):
    from sparse_long_context_lh_amd.binding import REGIONS
    for shape in [(65536, 16, 128, 3, 2, 1536, 0), (524288, 16, 128, 5, 4, 512, 0), (4096, 4, 64, 3, 2, 256, 1),
                  (1000, 2, 64, 1, 2, 0, 0)]:
        fwd, tot = L.lh_forward_workspace_bytes(*shape), L.lh_workspace_bytes(*shape)
        assert 0 < fwd < tot
        for name in REGIONS:
            off, nb = _region(L, shape, REGIONS.index(name))
            if name in ("dosub", "dqsub", "dksub", "dvsub"):   # written by lh_backward only
                assert off >= fwd
            else:                                               # lh_forward's context
                assert off + nb <= fwd
    shape = (4096, 4, 64, 3, 2, 256, 0)
    fwd, tot = L.lh_forward_workspace_bytes(*shape), L.lh_workspace_bytes(*shape)
    fake = 1 << 40  # never dereferenced: validation fails first
    assert L.lh_forward(fake, fake, fake, *shape, fake, fake, fwd - 1, None) == 2
    assert L.lh_backward(fake, *shape, fake, fake, fake, fake, fwd, None) == 2
    assert L.lh_backward(fake, *shape, fake, fake, fake, fake, tot - 1, None) == 2


def test_selection_hook_addresses(L):
    import ctypes
    from sparse_long_context_lh_amd.binding import REGIONS
    N, H, d, Lv, p, k = 524288, 16, 128, 5, 4, 512
    ws = 1 << 40  # an address only: lh_selection reads no memory
    off, nb = _region(L, (N, H, d, Lv, p, k, 0), REGIONS.index("sel"))
    assert nb == 4 * H * (Lv - 1) * k
    ptr = ctypes.c_void_p()
    for level in range(1, Lv):
        for dt in (0, 1):  # same place for either input type
            assert _region(L, (N, H, d, Lv, p, k, dt), REGIONS.index("sel"))[0] == off
        assert L.lh_selection(ws, N, H, d, Lv, p, k, level, ctypes.byref(ptr)) == 0
        assert ptr.value == ws + off + 4 * (level - 1) * H * k
    for bad_level in (0, Lv, -1):
        assert L.lh_selection(ws, N, H, d, Lv, p, k, bad_level, ctypes.byref(ptr)) == 1
        assert ptr.value is None
    assert L.lh_selection(ws, N, H, d, Lv, p, k, 1, None) == 1
    assert L.lh_selection(ws + 16, N, H, d, Lv, p, k, 1, ctypes.byref(ptr)) == 1   # misaligned ws
    assert L.lh_selection(None, N, H, d, Lv, p, k, 1, ctypes.byref(ptr)) == 1
    assert L.lh_selection(ws, 4096, 2, 64, 1, 2, 0, 1, ctypes.byref(ptr)) == 1     # L = 1: nothing selected
    assert L.lh_selection(ws, 4098, 2, 64, 3, 2, 4, 1, ctypes.byref(ptr)) == 1     # bad shape


def test_static_forward_validates_before_any_device_call(L):
    # rejections come before the scratch is looked up on a device
    assert L.lh_static_scratch_bytes() == 64 << 20
    fake = 1 << 40
    big = (65536, 16, 128, 3, 2, 1536, 0)      # forward workspace 1.3 GiB > 64 MiB
    assert L.lh_forward_workspace_bytes(*big) > L.lh_static_scratch_bytes()
    assert L.lh_forward_static(fake, fake, fake, *big, fake, None) == 2
    assert L.lh_forward_static(fake, fake, fake, 4098, 4, 64, 3, 2, 256, 0, fake, None) == 1
    assert L.lh_forward_static(None, fake, fake, 4096, 4, 64, 3, 2, 256, 0, fake, None) == 1
    assert L.lh_forward_static(fake, fake, fake, 4096, 4, 64, 3, 2, 256, 0, fake + 8, None) == 1


def test_ds_tile_budget_sizes_the_workspace(L):
    shape = (524288, 16, 128, 5, 4, 512, 0)
    S_pad = L.lh_padded_subseq_len(524288, 5, 4, 512)
    T = S_pad // 32
    tiles = 2 * 16 * (T * (T + 1) // 2) * 1024
    old = L.lh_ds_tile_budget()
    assert old == 32 << 30
    full = L.lh_workspace_bytes(*shape)
    fwd = L.lh_forward_workspace_bytes(*shape)
    try:
        L.lh_set_ds_tile_budget(0)
        small = L.lh_workspace_bytes(*shape)
        assert L.lh_forward_workspace_bytes(*shape) == fwd
        # the dS tiles are the last region: exactly their bytes (rounded to 256) go
        assert full - small == (tiles + 255) // 256 * 256
        L.lh_set_ds_tile_budget(tiles)       # exactly enough: kept
        assert L.lh_workspace_bytes(*shape) == full
        L.lh_set_ds_tile_budget(tiles - 1)   # one byte short: recomputed
        assert L.lh_workspace_bytes(*shape) == small
    finally:
        L.lh_set_ds_tile_budget(old)
    # dense attention over 512K tokens (L = 1): the tiles would take 4.4 TB;
    # the plan recomputes instead and the workspace is O(H S d)
    dense = L.lh_workspace_bytes(524288, 16, 128, 1, 2, 0, 0)
    assert 0 < dense < 200 << 30


def test_scored_forward_rejects_unknown_scorer(L):
    fake = 1 << 40
    shape = (4096, 4, 64, 3, 2, 256, 0)
    need = L.lh_workspace_bytes(*shape)
    assert L.lh_forward_scored(fake, fake, fake, *shape, 4, fake, fake, need, None) == 1
    assert L.lh_forward_scored(fake, fake, fake, *shape, -1, fake, fake, need, None) == 1
    assert L.lh_forward_scored(fake, fake, fake, 4098, 4, 64, 3, 2, 256, 0, 1, fake, fake, need, None) == 1
