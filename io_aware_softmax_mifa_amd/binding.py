"""Thin ctypes binding of libmifa (C ABI in include/mifa.h).

Argument marshalling only: every step of attention and of the row softmax runs in the HIP
library.  torch supplies
device memory and the current stream.  If the library is missing this module raises at import
time; there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

# MIFA_LIBRARY may name another build of the same library (the host-ASan test build).
_LIB_PATH = os.environ.get("MIFA_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmifa.so")

MIFA_OK = 0
STATUS_NAMES = {
    0: "MIFA_OK",
    1: "MIFA_ERR_NULL_POINTER",
    2: "MIFA_ERR_BAD_SHAPE",
    3: "MIFA_ERR_UNSUPPORTED_D",
    4: "MIFA_ERR_MISALIGNED",
    5: "MIFA_ERR_BAD_SCALE",
    6: "MIFA_ERR_TOO_LARGE",
    7: "MIFA_ERR_HIP",
    8: "MIFA_ERR_BAD_DTYPE",
    9: "MIFA_ERR_WORKSPACE",
    10: "MIFA_ERR_BAD_STRIDE",
    11: "MIFA_ERR_SCRATCH",
}
MIFA_DTYPE_BF16, MIFA_DTYPE_F32 = 0, 1
EXPORTED = ("mifa_fwd", "mifa_attention", "mifa_attention_strided", "mifa_attention_splitkv",
            "mifa_attention_splitkv_noalloc",
            "mifa_splitkv_workspace_bytes", "mifa_bwd", "mifa_bwd_strided", "mifa_bwd_workspace_bytes",
            "mifa_softmax_rows", "mifa_clock_probe", "mifa_status_string", "mifa_version",
            "mifa_last_hip_error")


class MifaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"libmifa.so not found at {_LIB_PATH}; build it with "
            "`python -m io_aware_softmax_mifa_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(_LIB_PATH)
    lib.mifa_fwd.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 4 + [ctypes.c_int, ctypes.c_float,
                                                                             ctypes.c_void_p]
    lib.mifa_fwd.restype = ctypes.c_int
    lib.mifa_attention.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 5 + [ctypes.c_int, ctypes.c_float,
                                                                                   ctypes.c_void_p]
    lib.mifa_attention.restype = ctypes.c_int
    lib.mifa_attention_splitkv.argtypes = ([ctypes.c_void_p] * 5 + [ctypes.c_int64] * 5 +
                                           [ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_int64,
                                            ctypes.c_void_p])
    lib.mifa_attention_splitkv.restype = ctypes.c_int
    lib.mifa_attention_splitkv_noalloc.argtypes = ([ctypes.c_void_p] * 5 + [ctypes.c_int64] * 5 +
                                                   [ctypes.c_int, ctypes.c_float, ctypes.c_void_p])
    lib.mifa_attention_splitkv_noalloc.restype = ctypes.c_int
    lib.mifa_splitkv_workspace_bytes.argtypes = [ctypes.c_int64] * 5
    lib.mifa_splitkv_workspace_bytes.restype = ctypes.c_int64
    lib.mifa_bwd.argtypes = ([ctypes.c_void_p] * 9 + [ctypes.c_int64] * 5 +
                             [ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p])
    lib.mifa_bwd.restype = ctypes.c_int
    lib.mifa_attention_strided.argtypes = ([ctypes.c_void_p] * 5 + [ctypes.c_int64] * 5 +
                                           [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                            ctypes.c_void_p])
    lib.mifa_attention_strided.restype = ctypes.c_int
    lib.mifa_bwd_strided.argtypes = ([ctypes.c_void_p] * 9 + [ctypes.c_int64] * 5 +
                                     [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                      ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p])
    lib.mifa_bwd_strided.restype = ctypes.c_int
    lib.mifa_bwd_workspace_bytes.argtypes = [ctypes.c_int64] * 3
    lib.mifa_bwd_workspace_bytes.restype = ctypes.c_int64
    lib.mifa_softmax_rows.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64] * 2 + [ctypes.c_int, ctypes.c_float,
                                                                                      ctypes.c_void_p]
    lib.mifa_softmax_rows.restype = ctypes.c_int
    lib.mifa_clock_probe.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(ctypes.c_int), ctypes.c_void_p]
    lib.mifa_clock_probe.restype = ctypes.c_int
    lib.mifa_status_string.argtypes = [ctypes.c_int]
    lib.mifa_status_string.restype = ctypes.c_char_p
    lib.mifa_version.argtypes = []
    lib.mifa_version.restype = ctypes.c_char_p
    lib.mifa_last_hip_error.argtypes = []
    lib.mifa_last_hip_error.restype = ctypes.c_int
    return lib


_lib = _load()


def library_path() -> str:
    return _LIB_PATH


def mifa_status_string(status: int) -> str:
    return _lib.mifa_status_string(int(status)).decode()


def mifa_version() -> str:
    return _lib.mifa_version().decode()


def mifa_last_hip_error() -> int:
    return int(_lib.mifa_last_hip_error())


def _ptr(t) -> int:
    if t is None:
        return 0
    if isinstance(t, int):
        return t
    return t.data_ptr()


def mifa_fwd_raw(q, k, v, o, lse, B, H, N, d, causal, scale, stream) -> int:
    """Call the C entry point with raw integer pointers or tensors; returns the status code."""
    return int(_lib.mifa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(N), int(d),
                             1 if causal else 0, float(scale), stream or None))


def mifa_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, stream=None) -> None:
    """Same arguments as the C function; tensors or integer device pointers.  Raises MifaError."""
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    st = mifa_fwd_raw(q, k, v, o, lse, B, H, N, d, causal, scale, stream)
    if st != MIFA_OK:
        extra = f" (hipError {mifa_last_hip_error()})" if st == 7 else ""
        raise MifaError(st, mifa_status_string(st) + extra)


def _raise(st):
    if st != MIFA_OK:
        extra = f" (hipError {mifa_last_hip_error()})" if st == 7 else ""
        raise MifaError(st, mifa_status_string(st) + extra)


def mifa_attention_raw(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, stream) -> int:
    return int(_lib.mifa_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(Nq), int(Nk),
                                   int(d), 1 if causal else 0, float(scale), stream or None))


def mifa_attention_splitkv_raw(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, workspace, workspace_bytes,
                               stream) -> int:
    return int(_lib.mifa_attention_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(Nq),
                                           int(Nk), int(d), 1 if causal else 0, float(scale), _ptr(workspace),
                                           int(workspace_bytes), stream or None))


def mifa_attention_splitkv_noalloc_raw(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, stream) -> int:
    """The allocation-free split-KV entry point (partials in the library's static device array)."""
    return int(_lib.mifa_attention_splitkv_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H),
                                                   int(Nq), int(Nk), int(d), 1 if causal else 0, float(scale),
                                                   stream or None))


def mifa_clock_probe_raw(out, span_us, stream) -> tuple[int, int]:
    """Launch the engine-clock probe on `stream`; returns (status, real-time counter rate in kHz).
    `out`: 32 int64 on the device, filled when the probe has run."""
    khz = ctypes.c_int(0)
    st = int(_lib.mifa_clock_probe(_ptr(out), int(span_us), ctypes.byref(khz), stream or None))
    return st, int(khz.value)


def mifa_splitkv_workspace_bytes(B, H, Nq, Nk, d) -> int:
    return int(_lib.mifa_splitkv_workspace_bytes(int(B), int(H), int(Nq), int(Nk), int(d)))


def _strides_array(strides):
    """A host int64 array for the strides argument, or a plain integer address (tests)."""
    if strides is None or isinstance(strides, int):
        return strides or None
    return (ctypes.c_int64 * len(strides))(*[int(x) for x in strides])


def mifa_attention_strided_raw(q, k, v, o, lse, B, H, Nq, Nk, d, strides, o_dtype, causal, scale, stream) -> int:
    """Call the C entry point; `strides`: 12 ints (batch, head, row strides of q, k, v, o)."""
    return int(_lib.mifa_attention_strided(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(Nq),
                                           int(Nk), int(d), _strides_array(strides), int(o_dtype),
                                           1 if causal else 0, float(scale), stream or None))


def mifa_bwd_strided_raw(q, k, v, o, lse, do, dq, dk, dv, B, H, Nq, Nk, d, strides, o_dtype, grad_dtype, causal,
                         scale, workspace, workspace_bytes, stream) -> int:
    """Call the C entry point; `strides`: 24 ints (q, k, v, o, dO, dq, dk, dv)."""
    return int(_lib.mifa_bwd_strided(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk),
                                     _ptr(dv), int(B), int(H), int(Nq), int(Nk), int(d), _strides_array(strides),
                                     int(o_dtype), int(grad_dtype), 1 if causal else 0, float(scale),
                                     _ptr(workspace), int(workspace_bytes), stream or None))


def _bhn(t):
    """(batch, head, row) strides of a [B, H, N, d] tensor whose d is contiguous."""
    return list(t.stride()[:3])


def _dense_bhnd(t) -> bool:
    return t.is_contiguous()


def _check(name, t, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != torch.bfloat16:
        raise ValueError(f"{name} must be bfloat16, got {t.dtype}")
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B, H, N, d]")
    if t.dim() == 4 and t.shape[3] > 1 and t.stride(3) != 1:
        raise ValueError(f"{name} must have its last (d) dimension contiguous")
    if shape is not None and tuple(t.shape) != shape:
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")


_MIFA_DTYPES = {torch.float32: 1, torch.bfloat16: 0}


def _outputs(q, out, lse, out_dtype=torch.float32):
    B, H, Nq, d = q.shape
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype not in _MIFA_DTYPES or out.device != q.device or out.stride(3) != 1:
        raise ValueError("out must be a float32 or bfloat16 tensor shaped like q on q's device, d contiguous")
    if lse.shape != (B, H, Nq) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 [B, H, Nq] tensor on q's device")
    return out, lse


def _qkv(q, k, v):
    _check("q", q)
    _check("k", k)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if k.shape != (B, H, Nk, d):
        raise ValueError(f"k has shape {tuple(k.shape)}, expected {(B, H, Nk, d)}")
    _check("v", v, (B, H, Nk, d))
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")
    return B, H, Nq, Nk, d


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False, scale=None,
              out: torch.Tensor | None = None, lse: torch.Tensor | None = None, out_dtype=torch.float32):
    """Exact attention forward.  q: bf16 [B, H, Nq, d], k, v: bf16 [B, H, Nk, d] on the GPU
    (d = 64 or 128; causal needs Nq <= Nk, the queries being the last Nq positions).  Any
    (batch, head, row) strides are read in place (d contiguous, strides multiples of 8).

    Returns (O [B, H, Nq, d] of out_dtype -- float32 or bfloat16 --, LSE float32 [B, H, Nq]);
    both are allocated here unless given (`out` may be strided too).  The launch is
    asynchronous on torch's current stream."""
    B, H, Nq, Nk, d = _qkv(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, lse = _outputs(q, out, lse, out_dtype)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        if all(_dense_bhnd(t) for t in (q, k, v, out)) and out.dtype == torch.float32:
            if Nq == Nk:
                mifa_fwd(q, k, v, out, lse, B, H, Nq, d, causal, scale, stream)
            else:
                _raise(mifa_attention_raw(q, k, v, out, lse, B, H, Nq, Nk, d, causal, scale, stream))
        else:
            strides = _bhn(q) + _bhn(k) + _bhn(v) + _bhn(out)
            _raise(mifa_attention_strided_raw(q, k, v, out, lse, B, H, Nq, Nk, d, strides, _MIFA_DTYPES[out.dtype],
                                              causal, scale, stream))
    return out, lse


def attention_splitkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False, scale=None,
                      out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None):
    """attention() with each head's keys split into ranges processed in parallel and merged
    by LSE (for few queries against many keys).  Contiguous tensors and float32 O only.
    `workspace`: a GPU tensor of at least mifa_splitkv_workspace_bytes(...) bytes, allocated
    here (uint8) unless given."""
    B, H, Nq, Nk, d = _qkv(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, lse = _outputs(q, out, lse)
    if not all(_dense_bhnd(t) for t in (q, k, v, out)) or out.dtype != torch.float32:
        raise ValueError("the split-KV path takes contiguous q, k, v and a contiguous float32 out")
    need = mifa_splitkv_workspace_bytes(B, H, Nq, Nk, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    nbytes = workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        _raise(mifa_attention_splitkv_raw(q, k, v, out, lse, B, H, Nq, Nk, d, causal, scale, workspace, nbytes,
                                          torch.cuda.current_stream(q.device).cuda_stream))
    return out, lse


# ---- the backward ---------------------------------------------------------------------------

def mifa_bwd_raw(q, k, v, o, lse, do, dq, dk, dv, B, H, Nq, Nk, d, causal, scale, workspace, workspace_bytes,
                 stream) -> int:
    """Call the C entry point with raw integer pointers or tensors; returns the status code."""
    return int(_lib.mifa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv),
                             int(B), int(H), int(Nq), int(Nk), int(d), 1 if causal else 0, float(scale),
                             _ptr(workspace), int(workspace_bytes), stream or None))


def mifa_bwd_workspace_bytes(B, H, Nq) -> int:
    return int(_lib.mifa_bwd_workspace_bytes(int(B), int(H), int(Nq)))


def attention_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
                       do: torch.Tensor, causal: bool = False, scale=None, workspace: torch.Tensor | None = None,
                       grad_dtype=torch.float32, grads=None):
    """Gradients (dq, dk, dv) of attention(q, k, v, causal, scale) for the upstream gradient
    do (bf16, shaped like q); o (float32 or bf16) and lse are that forward's outputs.  Any
    (batch, head, row) strides are read in place (d contiguous).  The gradients are allocated
    here, dense and of grad_dtype (float32 or bfloat16), unless `grads` = (dq, dk, dv) is
    given (any strides, one of those two types).  `workspace`: a GPU tensor of at least
    mifa_bwd_workspace_bytes(B, H, Nq) bytes, allocated here (uint8) unless given.
    Asynchronous on torch's current stream."""
    B, H, Nq, Nk, d = _qkv(q, k, v)
    _check("do", do, (B, H, Nq, d))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if (tuple(o.shape) != (B, H, Nq, d) or o.dtype not in _MIFA_DTYPES or o.device != q.device
            or o.stride(3) != 1):
        raise ValueError("o must be a float32 or bfloat16 [B, H, Nq, d] tensor on q's device, d contiguous")
    if tuple(lse.shape) != (B, H, Nq) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 [B, H, Nq] tensor on q's device")
    if grads is None:
        grads = (torch.empty((B, H, Nq, d), dtype=grad_dtype, device=q.device),
                 torch.empty((B, H, Nk, d), dtype=grad_dtype, device=q.device),
                 torch.empty((B, H, Nk, d), dtype=grad_dtype, device=q.device))
    dq, dk, dv = grads
    for name, g, shape in (("dq", dq, (B, H, Nq, d)), ("dk", dk, (B, H, Nk, d)), ("dv", dv, (B, H, Nk, d))):
        if tuple(g.shape) != shape or g.dtype != dq.dtype or g.dtype not in _MIFA_DTYPES or g.stride(3) != 1:
            raise ValueError(f"{name} must be a {shape} tensor of one type (float32 or bfloat16), d contiguous")
    need = mifa_bwd_workspace_bytes(B, H, Nq)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    nbytes = workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        if all(_dense_bhnd(t) for t in (q, k, v, o, do, dq, dk, dv)) and o.dtype == dq.dtype == torch.float32:
            _raise(mifa_bwd_raw(q, k, v, o, lse, do, dq, dk, dv, B, H, Nq, Nk, d, causal, scale, workspace, nbytes,
                                stream))
        else:
            strides = sum((_bhn(t) for t in (q, k, v, o, do, dq, dk, dv)), [])
            _raise(mifa_bwd_strided_raw(q, k, v, o, lse, do, dq, dk, dv, B, H, Nq, Nk, d, strides,
                                        _MIFA_DTYPES[o.dtype], _MIFA_DTYPES[dq.dtype], causal, scale, workspace,
                                        nbytes, stream))
    return dq, dk, dv


# ---- the row softmax ------------------------------------------------------------------------

_DTYPES = {torch.bfloat16: MIFA_DTYPE_BF16, torch.float32: MIFA_DTYPE_F32}


def mifa_softmax_rows_raw(x, y, lse, rows, cols, dtype, scale, stream) -> int:
    """Call the C entry point with raw integer pointers or tensors; returns the status code."""
    return int(_lib.mifa_softmax_rows(_ptr(x), _ptr(y), _ptr(lse), int(rows), int(cols), int(dtype), float(scale),
                                      stream or None))


def mifa_softmax_rows(x, y, lse, rows, cols, dtype, scale, stream=None) -> None:
    """Same arguments as the C function; tensors or integer device pointers.  Raises MifaError."""
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    st = mifa_softmax_rows_raw(x, y, lse, rows, cols, dtype, scale, stream)
    if st != MIFA_OK:
        extra = f" (hipError {mifa_last_hip_error()})" if st == 7 else ""
        raise MifaError(st, mifa_status_string(st) + extra)


def softmax_rows(x: torch.Tensor, scale: float = 1.0, out: torch.Tensor | None = None,
                 lse: torch.Tensor | None = None, with_lse: bool = True):
    """Softmax over the last dimension of a contiguous bf16 or fp32 GPU tensor.

    Returns (y, lse): y like x (same dtype), lse float32 over the leading dimensions (None when
    with_lse is False).  `out` may be x itself (in place).  Asynchronous on the current stream."""
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda":
        raise ValueError("x must be a GPU tensor")
    if x.dtype not in _DTYPES:
        raise ValueError(f"x must be bfloat16 or float32, got {x.dtype}")
    if x.dim() < 1 or x.numel() == 0 or not x.is_contiguous():
        raise ValueError("x must be a non-empty contiguous tensor")
    cols = x.shape[-1]
    rows = x.numel() // cols
    if out is None:
        out = torch.empty_like(x)
    if out.shape != x.shape or out.dtype != x.dtype or not out.is_contiguous() or out.device != x.device:
        raise ValueError("out must be a contiguous tensor like x on x's device")
    if with_lse and lse is None:
        lse = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    if lse is not None and (lse.numel() != rows or lse.dtype != torch.float32 or not lse.is_contiguous()
                            or lse.device != x.device):
        raise ValueError("lse must be a contiguous float32 tensor with one value per row on x's device")
    with torch.cuda.device(x.device):
        mifa_softmax_rows(x, out, lse, rows, cols, _DTYPES[x.dtype], scale,
                          torch.cuda.current_stream(x.device).cuda_stream)
    return out, lse
