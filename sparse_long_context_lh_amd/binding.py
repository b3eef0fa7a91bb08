"""Thin ctypes binding of liblh.so (the C ABI in include/lh.h).

Argument marshalling only: every step of the layer runs in the HIP kernels of
liblh.so. PyTorch supplies device memory and the current HIP stream. Loading
fails loudly if the library has not been built; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblh.so")

LH_OK, LH_EINVAL, LH_EWORKSPACE, LH_EUNSUPPORTED, LH_EHIP = range(5)
DTYPES = {torch.bfloat16: 0, torch.float32: 1}
REGIONS = ["scores", "sel", "slot", "ent", "qhi", "qlo", "khi", "klo", "v", "qhi_t", "khi_t", "v_t",
           "osub", "lse", "dosub", "dqsub", "dksub", "dvsub"]
_REGION_DTYPE = {"scores": torch.float32, "sel": torch.int32, "slot": torch.int32, "ent": torch.int32,
                 "qhi": torch.float16, "qlo": torch.float16, "khi": torch.float16, "klo": torch.float16,
                 "v": torch.float16, "qhi_t": torch.float16, "khi_t": torch.float16, "v_t": torch.float16,
                 "osub": torch.float32, "lse": torch.float32, "dosub": torch.float32,
                 "dqsub": torch.float32, "dksub": torch.float32, "dvsub": torch.float32}

_lib = None


class LighthouseError(RuntimeError):
    """A non-OK status from the C ABI."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (what, strerror(status), status))


def lib() -> ctypes.CDLL:
    """The loaded liblh.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("liblh.so is not built (%s); run `python -m sparse_long_context_lh_amd.build` "
                          "or __graft_entry__.build()" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    i64, i32, sz, vp, u32 = ctypes.c_int64, ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_uint32
    shape = [i64, i32, i32, i32, i32, i32, i32]  # N, H, d, L, p, k, dtype
    sig = {
        "lh_strerror": (ctypes.c_char_p, [i32]),
        "lh_check_shape": (i32, shape),
        "lh_subseq_len": (i64, [i64, i32, i32, i32]),
        "lh_padded_subseq_len": (i64, [i64, i32, i32, i32]),
        "lh_workspace_bytes": (sz, shape),
        "lh_forward": (i32, [vp, vp, vp] + shape + [vp, vp, sz, vp]),
        "lh_backward": (i32, [vp] + shape + [vp, vp, vp, vp, sz, vp]),
        "lh_forward_timed": (i32, [vp, vp, vp] + shape + [vp, vp, sz, vp, vp]),
        "lh_backward_timed": (i32, [vp] + shape + [vp, vp, vp, vp, sz, vp, vp]),
        "lh_stage_count": (i32, [i32]),
        "lh_stage_name": (ctypes.c_char_p, [i32, i32]),
        "lh_region_info": (i32, shape + [i32, ctypes.POINTER(sz), ctypes.POINTER(sz)]),
        "lh_selftest_sqrt": (i32, [u32, u32, vp, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def strerror(status: int) -> str:
    return lib().lh_strerror(status).decode()


def _check(status: int, what: str) -> None:
    if status != LH_OK:
        raise LighthouseError(status, what)


def _dt(dtype: torch.dtype) -> int:
    if dtype not in DTYPES:
        raise TypeError("dtype must be torch.bfloat16 or torch.float32, got %s" % dtype)
    return DTYPES[dtype]


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def subseq_len(N: int, L: int, p: int, k: int) -> int:
    return lib().lh_subseq_len(N, L, p, k)


def padded_subseq_len(N: int, L: int, p: int, k: int) -> int:
    return lib().lh_padded_subseq_len(N, L, p, k)


def workspace_bytes(N, H, d, L, p, k, dtype) -> int:
    return lib().lh_workspace_bytes(N, H, d, L, p, k, _dt(dtype))


def check_shape(N, H, d, L, p, k, dtype) -> int:
    return lib().lh_check_shape(N, H, d, L, p, k, _dt(dtype))


def alloc_workspace(N, H, d, L, p, k, dtype, device="cuda") -> torch.Tensor:
    n = workspace_bytes(N, H, d, L, p, k, dtype)
    if n == 0:
        _check(check_shape(N, H, d, L, p, k, dtype), "workspace size")
    return torch.empty(n, dtype=torch.uint8, device=device)


def _shape_of(x: torch.Tensor):
    if x.dim() != 3 or not x.is_contiguous() or not x.is_cuda:
        raise ValueError("expected a contiguous [H, N, d] CUDA tensor")
    H, N, d = x.shape
    return N, H, d


def forward(q, k, v, L: int, p: int, k_sel: int, ws: torch.Tensor | None = None,
            out: torch.Tensor | None = None, stream=None, events=None):
    """Lighthouse forward on [H, N, d] tensors; returns (out, ws)."""
    N, H, d = _shape_of(q)
    for t in (k, v):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous():
            raise ValueError("q, k, v must share shape, dtype and be contiguous")
    dt = _dt(q.dtype)
    if ws is None:
        ws = alloc_workspace(N, H, d, L, p, k_sel, q.dtype, q.device)
    if out is None:
        out = torch.empty_like(q)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), N, H, d, L, p, k_sel, dt,
            out.data_ptr(), ws.data_ptr(), ws.numel(), _stream(stream))
    if events is None:
        _check(lib().lh_forward(*args), "lh_forward")
    else:
        _check(lib().lh_forward_timed(*args, events), "lh_forward_timed")
    return out, ws


def backward(dout, L: int, p: int, k_sel: int, ws: torch.Tensor, dq=None, dk=None, dv=None,
             stream=None, events=None):
    """Lighthouse backward (indices of the preceding forward held fixed); returns (dq, dk, dv)."""
    N, H, d = _shape_of(dout)
    dt = _dt(dout.dtype)
    dq = torch.empty_like(dout) if dq is None else dq
    dk = torch.empty_like(dout) if dk is None else dk
    dv = torch.empty_like(dout) if dv is None else dv
    args = (dout.data_ptr(), N, H, d, L, p, k_sel, dt, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
            ws.data_ptr(), ws.numel(), _stream(stream))
    if events is None:
        _check(lib().lh_backward(*args), "lh_backward")
    else:
        _check(lib().lh_backward_timed(*args, events), "lh_backward_timed")
    return dq, dk, dv


def region(ws: torch.Tensor, name: str, N, H, d, L, p, k, dtype) -> torch.Tensor:
    """A typed, flat view of one intermediate inside the workspace."""
    off, nbytes = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().lh_region_info(N, H, d, L, p, k, _dt(dtype), REGIONS.index(name),
                                ctypes.byref(off), ctypes.byref(nbytes)), "lh_region_info")
    return ws[off.value:off.value + nbytes.value].view(_REGION_DTYPE[name])


def stage_names(backward: bool) -> list[str]:
    n = lib().lh_stage_count(int(backward))
    return [lib().lh_stage_name(int(backward), i).decode() for i in range(n)]


def selftest_sqrt(first: int, count: int, stream=None) -> int:
    """Number of fp32 inputs in [first, first+count) whose device sqrtf is not correctly rounded."""
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    _check(lib().lh_selftest_sqrt(first, count, cnt.data_ptr(), _stream(stream)), "lh_selftest_sqrt")
    return int(cnt.item())
