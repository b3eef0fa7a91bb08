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
SCORERS = ("sum", "product", "query", "key")  # lh_scorer, in order
REGIONS = ["scores", "sel", "slot", "ent", "qhi", "qlo", "khi", "klo", "v", "qhi_t", "khi_t", "v_t",
           "osub", "lse", "dosub", "dqsub", "dksub", "dvsub", "exp"]
_REGION_DTYPE = {"scores": torch.float32, "sel": torch.int32, "slot": torch.int32, "ent": torch.int32,
                 "qhi": torch.float16, "qlo": torch.float16, "khi": torch.float16, "klo": torch.float16,
                 "v": torch.float16, "qhi_t": torch.float16, "khi_t": torch.float16, "v_t": torch.float16,
                 "osub": torch.float32, "lse": torch.float32, "dosub": torch.float32,
                 "dqsub": torch.float32, "dksub": torch.float32, "dvsub": torch.float32, "exp": torch.int32}

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
        "lh_forward_workspace_bytes": (sz, shape),
        "lh_selection": (i32, [vp, i64, i32, i32, i32, i32, i32, i32, ctypes.POINTER(vp)]),
        "lh_forward": (i32, [vp, vp, vp] + shape + [vp, vp, sz, vp]),
        "lh_backward": (i32, [vp] + shape + [vp, vp, vp, vp, sz, vp]),
        "lh_forward_timed": (i32, [vp, vp, vp] + shape + [vp, vp, sz, vp, vp]),
        "lh_forward_static": (i32, [vp, vp, vp] + shape + [vp, vp]),
        "lh_forward_scored": (i32, [vp, vp, vp] + shape + [i32, vp, vp, sz, vp]),
        "lh_forward_nograd": (i32, [vp, vp, vp] + shape + [vp, vp, sz, vp]),
        "lh_forward_nograd_timed": (i32, [vp, vp, vp] + shape + [vp, vp, sz, vp, vp]),
        "lh_static_scratch_bytes": (sz, []),
        "lh_set_ds_tile_budget": (None, [sz]),
        "lh_layer_workspace_bytes": (sz, [i64, i32, i32, i32, i32, i32, i32, i32]),
        "lh_layer_forward": (i32, [vp, vp, i64, i32, i32, i32, i32, i32, i32, i32, vp, vp, sz, vp]),
        "lh_layer_backward": (i32, [vp, vp, vp, i64, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, sz, vp]),
        "lh_ds_tile_budget": (sz, []),
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


def forward_workspace_bytes(N, H, d, L, p, k, dtype) -> int:
    return lib().lh_forward_workspace_bytes(N, H, d, L, p, k, _dt(dtype))


def check_shape(N, H, d, L, p, k, dtype) -> int:
    return lib().lh_check_shape(N, H, d, L, p, k, _dt(dtype))


def alloc_workspace(N, H, d, L, p, k, dtype, device="cuda", forward_only=False) -> torch.Tensor:
    """A workspace for lh_forward + lh_backward (forward_only: lh_forward alone)."""
    n = (forward_workspace_bytes if forward_only else workspace_bytes)(N, H, d, L, p, k, dtype)
    if n == 0:
        _check(check_shape(N, H, d, L, p, k, dtype), "workspace size")
    return torch.empty(n, dtype=torch.uint8, device=device)


def _shape_of(x: torch.Tensor):
    if x.dim() != 3 or not x.is_contiguous() or not x.is_cuda:
        raise ValueError("expected a contiguous [H, N, d] CUDA tensor")
    H, N, d = x.shape
    return N, H, d


def _like(t: torch.Tensor, ref: torch.Tensor, what: str) -> None:
    """A caller-supplied output must match ref in shape, dtype and device and be contiguous."""
    if t.shape != ref.shape or t.dtype != ref.dtype or t.device != ref.device or not t.is_contiguous():
        raise ValueError("%s must be a contiguous %s tensor of shape %s on %s" % (what, ref.dtype, tuple(ref.shape),
                                                                                ref.device))


def _check_ws(ws: torch.Tensor, ref: torch.Tensor) -> None:
    if ws.dtype != torch.uint8 or ws.dim() != 1 or not ws.is_contiguous() or ws.device != ref.device:
        raise ValueError("ws must be a contiguous 1-D uint8 tensor on %s" % ref.device)


def forward(q, k, v, L: int, p: int, k_sel: int, ws: torch.Tensor | None = None,
            out: torch.Tensor | None = None, stream=None, events=None, scorer: str = "sum"):
    """Lighthouse forward on [H, N, d] tensors; returns (out, ws). `scorer`
    picks the level-0 score ("sum", "product", "query", "key")."""
    N, H, d = _shape_of(q)
    for t in (k, v):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous():
            raise ValueError("q, k, v must share shape, dtype and be contiguous")
    dt = _dt(q.dtype)
    if ws is None:
        ws = alloc_workspace(N, H, d, L, p, k_sel, q.dtype, q.device)
    _check_ws(ws, q)
    if out is None:
        out = torch.empty_like(q)
    _like(out, q, "out")
    if scorer not in SCORERS:
        raise ValueError("scorer must be one of %s" % (SCORERS,))
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), N, H, d, L, p, k_sel, dt,
            out.data_ptr(), ws.data_ptr(), ws.numel(), _stream(stream))
    if scorer != "sum":
        if events is not None:
            raise ValueError("timed calls use the default scorer")
        _check(lib().lh_forward_scored(*args[:10], SCORERS.index(scorer), *args[10:]), "lh_forward_scored")
    elif events is None:
        _check(lib().lh_forward(*args), "lh_forward")
    else:
        _check(lib().lh_forward_timed(*args, events), "lh_forward_timed")
    return out, ws


def forward_nograd(q, k, v, L: int, p: int, k_sel: int, ws: torch.Tensor | None = None,
                   out: torch.Tensor | None = None, stream=None, events=None):
    """lh_forward_nograd: the forward for calls no backward follows; returns
    (out, ws). A new workspace is sized for the forward alone."""
    N, H, d = _shape_of(q)
    for t in (k, v):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous():
            raise ValueError("q, k, v must share shape, dtype and be contiguous")
    if ws is None:
        ws = alloc_workspace(N, H, d, L, p, k_sel, q.dtype, q.device, forward_only=True)
    _check_ws(ws, q)
    if out is None:
        out = torch.empty_like(q)
    _like(out, q, "out")
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), N, H, d, L, p, k_sel, _dt(q.dtype),
            out.data_ptr(), ws.data_ptr(), ws.numel(), _stream(stream))
    if events is None:
        _check(lib().lh_forward_nograd(*args), "lh_forward_nograd")
    else:
        _check(lib().lh_forward_nograd_timed(*args, events), "lh_forward_nograd_timed")
    return out, ws


def forward_static(q, k, v, L: int, p: int, k_sel: int, out: torch.Tensor | None = None, stream=None):
    """Lighthouse forward that uses the library's static device scratch as its
    workspace (no allocation inside the call); returns out."""
    N, H, d = _shape_of(q)
    for t in (k, v):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous():
            raise ValueError("q, k, v must share shape, dtype and be contiguous")
    if out is None:
        out = torch.empty_like(q)
    _like(out, q, "out")
    _check(lib().lh_forward_static(q.data_ptr(), k.data_ptr(), v.data_ptr(), N, H, d, L, p, k_sel, _dt(q.dtype),
                                   out.data_ptr(), _stream(stream)), "lh_forward_static")
    return out


def layer_workspace_bytes(N, H, d, d_model, L, p, k, dtype) -> int:
    return lib().lh_layer_workspace_bytes(N, H, d, d_model, L, p, k, _dt(dtype))


def layer_forward(x, w_qkv, H: int, d: int, L: int, p: int, k_sel: int, ws=None, out=None, stream=None):
    """Projections of x [N, d_model] by w_qkv [d_model, 3 H d], then the layer;
    returns (out [H, N, d], ws)."""
    if x.dim() != 2 or not x.is_contiguous() or not x.is_cuda:
        raise ValueError("x must be a contiguous [N, d_model] CUDA tensor")
    N, dm = x.shape
    if w_qkv.shape != (dm, 3 * H * d) or w_qkv.dtype != x.dtype or not w_qkv.is_contiguous():
        raise ValueError("w_qkv must be a contiguous [d_model, 3 H d] tensor of x's dtype")
    if ws is None:
        n = layer_workspace_bytes(N, H, d, dm, L, p, k_sel, x.dtype)
        if n == 0:
            _check(check_shape(N, H, d, L, p, k_sel, x.dtype) or LH_EUNSUPPORTED, "layer workspace size")
        ws = torch.empty(n, dtype=torch.uint8, device=x.device)
    _check_ws(ws, x)
    if out is None:
        out = torch.empty(H, N, d, dtype=x.dtype, device=x.device)
    if out.shape != (H, N, d) or out.dtype != x.dtype or not out.is_contiguous() or out.device != x.device:
        raise ValueError("out must be a contiguous [H, N, d] tensor of x's dtype")
    _check(lib().lh_layer_forward(x.data_ptr(), w_qkv.data_ptr(), N, H, d, dm, L, p, k_sel, _dt(x.dtype),
                                  out.data_ptr(), ws.data_ptr(), ws.numel(), _stream(stream)), "lh_layer_forward")
    return out, ws


def layer_backward(x, w_qkv, dout, H: int, d: int, L: int, p: int, k_sel: int, ws, dx=None, dw=None, stream=None):
    """dx [N, d_model] and dw [d_model, 3 H d] of the layer with its
    projections (indices of the preceding layer_forward held fixed)."""
    N, dm = x.shape
    if dout.shape != (H, N, d) or dout.dtype != x.dtype or not dout.is_contiguous():
        raise ValueError("dout must be a contiguous [H, N, d] tensor of x's dtype")
    dx = torch.empty_like(x) if dx is None else dx
    dw = torch.empty_like(w_qkv) if dw is None else dw
    _like(dx, x, "dx")
    _like(dw, w_qkv, "dw")
    _check_ws(ws, x)
    _check(lib().lh_layer_backward(x.data_ptr(), w_qkv.data_ptr(), dout.data_ptr(), N, H, d, dm, L, p, k_sel,
                                   _dt(x.dtype), dx.data_ptr(), dw.data_ptr(), ws.data_ptr(), ws.numel(),
                                   _stream(stream)), "lh_layer_backward")
    return dx, dw


def layer_qkv(ws: torch.Tensor, N: int, H: int, d: int, dtype) -> torch.Tensor:
    """The projected rows [3, H, N, d] lh_layer_forward leaves at the start of ws."""
    nb = 3 * H * N * d * (2 if dtype == torch.bfloat16 else 4)
    return ws[:nb].view(dtype).view(3, H, N, d)


def set_ds_tile_budget(nbytes: int) -> None:
    """Largest share of a workspace the backward's stored dS tiles may take
    (0: the dQ kernel always recomputes S and dP)."""
    lib().lh_set_ds_tile_budget(nbytes)


def ds_tile_budget() -> int:
    return lib().lh_ds_tile_budget()


def static_scratch_bytes() -> int:
    return lib().lh_static_scratch_bytes()


def backward(dout, L: int, p: int, k_sel: int, ws: torch.Tensor, dq=None, dk=None, dv=None,
             stream=None, events=None):
    """Lighthouse backward (indices of the preceding forward held fixed); returns (dq, dk, dv)."""
    N, H, d = _shape_of(dout)
    dt = _dt(dout.dtype)
    dq = torch.empty_like(dout) if dq is None else dq
    dk = torch.empty_like(dout) if dk is None else dk
    dv = torch.empty_like(dout) if dv is None else dv
    for t, what in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _like(t, dout, what)
    _check_ws(ws, dout)
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


def selection(ws: torch.Tensor, N, H, d, L, p, k, level: int) -> torch.Tensor:
    """The [H, k] selection of pyramid level `level` (1..L-1) that the last
    lh_forward on ws made, as a view of ws (lh_selection gives its address)."""
    ptr = ctypes.c_void_p()
    _check(lib().lh_selection(ws.data_ptr(), N, H, d, L, p, k, level, ctypes.byref(ptr)), "lh_selection")
    off = (ptr.value or 0) - ws.data_ptr()
    return ws[off:off + 4 * H * k].view(torch.int32).view(H, k)


def stage_names(backward: bool) -> list[str]:
    n = lib().lh_stage_count(int(backward))
    return [lib().lh_stage_name(int(backward), i).decode() for i in range(n)]


def selftest_sqrt(first: int, count: int, stream=None) -> int:
    """Number of fp32 inputs in [first, first+count) whose device sqrtf is not correctly rounded."""
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    _check(lib().lh_selftest_sqrt(first, count, cnt.data_ptr(), _stream(stream)), "lh_selftest_sqrt")
    return int(cnt.item())
