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
    fake = 1 << 40  # never dereferenced: validation fails first
    # bad shape
    assert L.lh_forward(fake, fake, fake, 4098, 4, 64, 3, 2, 256, 0, fake, fake, need, None) == 1
    # null input pointer
    assert L.lh_forward(None, fake, fake, *shape, fake, fake, need, None) == 1
    # misaligned output pointer
    assert L.lh_forward(fake, fake, fake, *shape, fake + 2, fake, need, None) == 1
    # workspace too small, null, misaligned
    assert L.lh_forward(fake, fake, fake, *shape, fake, fake, need - 1, None) == 2
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


def test_stage_names(L):
    from sparse_long_context_lh_amd import binding
    assert binding.stage_names(False) == ["front", "topk", "index", "gather", "attn_fwd", "scatter"]
    assert binding.stage_names(True) == ["scatter_bwd", "bwd_prep", "attn_bwd_dkdv", "attn_bwd_dq", "pool_bwd"]
