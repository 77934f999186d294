"""ctypes binding of libsdpa03.so (argument marshalling only).

Each function takes torch tensors that live on a ROCm device, reads their
pointers and strides, allocates outputs with torch, and calls the C entry
point of the same name on the current torch stream.  Every step of the
attention itself runs in the library's HIP kernels; if the library is not
built, the first call raises.
"""

from __future__ import annotations

import ctypes
import math
import os

import numpy as np
import torch

from .build import LIB_PATH

_DTYPE_CODES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
_BAD_DTYPE = 99  # lets the library report SDPA_ERR_DTYPE itself

STATUS_NAMES = {
    0: "SDPA_OK", 1: "SDPA_ERR_NULL", 2: "SDPA_ERR_DTYPE", 3: "SDPA_ERR_HEAD_DIM",
    4: "SDPA_ERR_SHAPE", 5: "SDPA_ERR_STRIDE", 6: "SDPA_ERR_ALIGN", 7: "SDPA_ERR_BATCH",
    8: "SDPA_ERR_SEQLEN", 9: "SDPA_ERR_SCALE", 10: "SDPA_ERR_HIP", 11: "SDPA_ERR_WORKSPACE",
    12: "SDPA_ERR_SCRATCH",
}

# Bytes of the static scratch attn_fwd_splitk_noalloc uses (sdpa03.h).
NOALLOC_SCRATCH_BYTES = 32 << 20

EXPORTED = (
    "sdpa_status_string",
    "attn_fwd",
    "attn_fwd_compact_varlen",
    "attn_fwd_padded_varlen",
    "attn_fwd_bias",
    "attn_fwd_compact_varlen_bias",
    "attn_fwd_padded_varlen_bias",
    "attn_fwd_splitk",
    "attn_fwd_splitk_noalloc",
    "sdpa_fwd_splitk_plan",
    "attn_bwd",
    "attn_bwd_compact_varlen",
    "attn_bwd_padded_varlen",
    "sdpa_bwd_workspace_bytes",
    "sdpa_check_cu_seqlens_host",
    "sdpa_kernel_config",
)


class SdpaError(RuntimeError):
    """A non-zero sdpa_status from the library."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_stride = ctypes.POINTER(ctypes.c_int64)
_i32p = ctypes.POINTER(ctypes.c_int32)


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load the shared library once and declare its signatures.

    The default is the in-tree build; SDPA03_LIBRARY names another build of
    the same library (the dispatch-table sweep uses it for its candidates).
    """
    global _lib
    if _lib is not None:
        return _lib
    path = path or os.environ.get("SDPA03_LIBRARY") or LIB_PATH
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is not built; build it with `python -m scaled_dot_product_03_amd.build` "
            "(or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    lib.sdpa_status_string.restype = ctypes.c_char_p
    lib.sdpa_status_string.argtypes = [ctypes.c_int]
    common_tail = [_stride, _stride, _stride, _stride, ctypes.c_float, _i32, _p]
    lib.attn_fwd.restype = ctypes.c_int
    lib.attn_fwd.argtypes = [_p, _p, _p, _p, _p, ctypes.c_int, _i32, _i32, _i32, _i32, _i32] + common_tail
    lib.attn_fwd_compact_varlen.restype = ctypes.c_int
    lib.attn_fwd_compact_varlen.argtypes = (
        [_p, _p, _p, _p, _p, ctypes.c_int, _i32, _i32, _i32, _i32, _i32, _p, _p, _i32, _i32, _i32]
        + common_tail)
    lib.attn_fwd_padded_varlen.restype = ctypes.c_int
    lib.attn_fwd_padded_varlen.argtypes = (
        [_p, _p, _p, _p, _p, ctypes.c_int, _i32, _i32, _i32, _i32, _i32, _p, _p] + common_tail)
    bias_tail = [_stride, _stride, _stride, _stride, _stride, ctypes.c_float, _i32, _p]
    lib.attn_fwd_bias.restype = ctypes.c_int
    lib.attn_fwd_bias.argtypes = (
        [_p, _p, _p, _p, _p, _p, ctypes.c_int, _i32, _i32, _i32, _i32, _i32] + bias_tail)
    lib.attn_fwd_compact_varlen_bias.restype = ctypes.c_int
    lib.attn_fwd_compact_varlen_bias.argtypes = (
        [_p, _p, _p, _p, _p, _p, ctypes.c_int, _i32, _i32, _i32, _i32, _i32, _p, _p, _i32, _i32,
         _i32] + bias_tail)
    lib.attn_fwd_padded_varlen_bias.restype = ctypes.c_int
    lib.attn_fwd_padded_varlen_bias.argtypes = (
        [_p, _p, _p, _p, _p, _p, ctypes.c_int, _i32, _i32, _i32, _i32, _i32, _p, _p] + bias_tail)
    lib.attn_fwd_splitk.restype = ctypes.c_int
    lib.attn_fwd_splitk.argtypes = (
        [_p, _p, _p, _p, _p, ctypes.c_int, _i32, _i32, _i32, _i32, _i32, _stride, _stride, _stride,
         _stride, ctypes.c_float, _i32, _i32, _p, ctypes.c_uint64, _p])
    lib.attn_fwd_splitk_noalloc.restype = ctypes.c_int
    lib.attn_fwd_splitk_noalloc.argtypes = (
        [_p, _p, _p, _p, _p, ctypes.c_int, _i32, _i32, _i32, _i32, _i32, _stride, _stride, _stride,
         _stride, ctypes.c_float, _i32, _i32, _p])
    lib.sdpa_fwd_splitk_plan.restype = ctypes.c_int
    lib.sdpa_fwd_splitk_plan.argtypes = [ctypes.c_int, _i32, _i32, _i32, _i32, _i32, _i32, _i32p,
                                         ctypes.POINTER(ctypes.c_uint64)]
    lib.attn_bwd.restype = ctypes.c_int
    lib.attn_bwd.argtypes = (
        [_p, _p, _p, _p, _p, _p, _p, _p, _p, ctypes.c_int, _i32, _i32, _i32, _i32, _i32,
         _stride, _stride, _stride, _stride, _stride, ctypes.c_float, _i32, _p, ctypes.c_uint64,
         _p])
    bwd_tail = [_stride, _stride, _stride, _stride, _stride, ctypes.c_float, _i32, _p,
                ctypes.c_uint64, _p]
    lib.attn_bwd_compact_varlen.restype = ctypes.c_int
    lib.attn_bwd_compact_varlen.argtypes = (
        [_p, _p, _p, _p, _p, _p, _p, _p, _p, ctypes.c_int, _i32, _i32, _i32, _i32, _i32, _p, _p,
         _i32, _i32, _i32] + bwd_tail)
    lib.attn_bwd_padded_varlen.restype = ctypes.c_int
    lib.attn_bwd_padded_varlen.argtypes = (
        [_p, _p, _p, _p, _p, _p, _p, _p, _p, ctypes.c_int, _i32, _i32, _i32, _i32, _i32, _p, _p]
        + bwd_tail)
    lib.sdpa_bwd_workspace_bytes.restype = ctypes.c_int
    lib.sdpa_bwd_workspace_bytes.argtypes = [_i32, _i32, _i32, ctypes.POINTER(ctypes.c_uint64)]
    lib.sdpa_check_cu_seqlens_host.restype = ctypes.c_int
    lib.sdpa_check_cu_seqlens_host.argtypes = [_i32p, _i32, _i32, _i32]
    lib.sdpa_kernel_config.restype = ctypes.c_int
    lib.sdpa_kernel_config.argtypes = [ctypes.c_int, _i32, _i32, _i32, _i32, _i32, _i32, _i32p,
                                       _i32p, _i32p]
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        msg = load_library().sdpa_status_string(status).decode()
        raise SdpaError(status, msg)


def _strides(t: torch.Tensor):
    return (ctypes.c_int64 * 4)(*t.stride())


def _dtype_code(t: torch.Tensor) -> int:
    return _DTYPE_CODES.get(t.dtype, _BAD_DTYPE)


def _stream_handle(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _scale(scale, head_dim):
    return 1.0 / math.sqrt(head_dim) if scale is None else float(scale)


def _require_gpu(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("inputs must be ROCm device tensors")


def kernel_config(dtype: torch.dtype, head_dim: int, seqlen_q: int, seqlen_k: int,
                  causal: bool = False, mode: int = 0, single_group: bool = False):
    """(block_m, block_n, waves) of the compiled forward kernel for these
    sizes (varlen: the longest sequence's lengths), mask and layout (mode 0
    dense, 1 compact, 2 padded); single_group for the forward with a bias
    and for the split forward (which uses causal=False, mode=0 for both
    masks)."""
    lib = load_library()
    bm, bn, w = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib.sdpa_kernel_config(_DTYPE_CODES.get(dtype, _BAD_DTYPE), head_dim, int(causal), mode,
                                  seqlen_q, seqlen_k, int(bool(single_group)), ctypes.byref(bm),
                                  ctypes.byref(bn), ctypes.byref(w)))
    return bm.value, bn.value, w.value


def check_cu_seqlens_host(cu, total: int, max_len: int) -> None:
    """Validate a host cu_seqlens array with the library's own check."""
    arr = np.ascontiguousarray(np.asarray(cu, dtype=np.int32))
    ptr = arr.ctypes.data_as(_i32p)
    _check(load_library().sdpa_check_cu_seqlens_host(ptr, arr.size - 1, int(total), int(max_len)))


def _outputs(q, out, lse, lse_shape):
    """The output O (q's shape, dtype and device; any strides the library
    accepts) and the fp32 logsumexp (contiguous, lse_shape) of a forward
    call: the caller's, checked before anything is launched, or new ones.
    The kernels write through these pointers, so a wrong size or type would
    write out of bounds or garble the result."""
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or out.device != q.device:
        raise ValueError(f"out must have the shape, dtype and device of q: got "
                         f"{tuple(out.shape)} {out.dtype} {out.device}, want {tuple(q.shape)} "
                         f"{q.dtype} {q.device}")
    if lse is None:
        lse = torch.empty(lse_shape, dtype=torch.float32, device=q.device)
    elif (tuple(lse.shape) != tuple(lse_shape) or lse.dtype != torch.float32
          or lse.device != q.device or not lse.is_contiguous()):
        raise ValueError(f"lse must be a contiguous float32 tensor of shape {tuple(lse_shape)} on "
                         f"{q.device}: got {tuple(lse.shape)} {lse.dtype} {lse.device}"
                         f"{'' if lse.is_contiguous() else ' (not contiguous)'}")
    return out, lse


def _bias_view(bias, q, shape):
    """The bias broadcast (stride 0, no copy) to the rank-4 score view."""
    if not bias.is_cuda or bias.device != q.device:
        raise ValueError("bias must be on the device of q")
    if bias.dtype != q.dtype:
        raise ValueError("bias must have the dtype of q")
    return bias.expand(*shape)


def attn_fwd(q, k, v, scale=None, causal=False, out=None, lse=None, bias=None):
    """Dense forward.  q: (B,H,Sq,D), k/v: (B,H,Sk,D) -> (o, lse (B,H,Sq) fp32).

    ``bias`` (optional, q's dtype, broadcastable to (B,H,Sq,Sk)) is added to
    the scaled scores."""
    lib = load_library()
    _require_gpu(q, k, v)
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    if k.shape != (B, H, Sk, D) or v.shape != k.shape:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must share one dtype")
    o, lse = _outputs(q, out, lse, (B, H, Sq))
    if bias is None:
        _check(lib.attn_fwd(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
            _dtype_code(q), B, H, Sq, Sk, D,
            _strides(q), _strides(k), _strides(v), _strides(o),
            _scale(scale, D), int(bool(causal)), _stream_handle(q.device)))
    else:
        bv = _bias_view(bias, q, (B, H, Sq, Sk))
        _check(lib.attn_fwd_bias(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), bv.data_ptr(), o.data_ptr(), lse.data_ptr(),
            _dtype_code(q), B, H, Sq, Sk, D,
            _strides(q), _strides(k), _strides(v), _strides(bv), _strides(o),
            _scale(scale, D), int(bool(causal)), _stream_handle(q.device)))
    return o, lse


def splitk_plan(dtype: torch.dtype, B: int, H: int, seqlen_q: int, seqlen_k: int, head_dim: int,
                num_splits: int = 0):
    """(splits used, workspace bytes) of a split forward with these sizes."""
    lib = load_library()
    used, nbytes = ctypes.c_int32(), ctypes.c_uint64()
    _check(lib.sdpa_fwd_splitk_plan(_DTYPE_CODES.get(dtype, _BAD_DTYPE), B, H, seqlen_q, seqlen_k,
                                    head_dim, int(num_splits), ctypes.byref(used),
                                    ctypes.byref(nbytes)))
    return used.value, nbytes.value


def attn_fwd_splitk(q, k, v, scale=None, causal=False, num_splits=0, out=None, lse=None,
                    workspace=None):
    """Key-parallel dense forward (same results as attn_fwd).

    q: (B,H,Sq,D), k/v: (B,H,Sk,D).  num_splits <= 0 lets the library pick.
    The workspace (a uint8 device tensor) is allocated here unless given.
    Returns (o, lse (B,H,Sq) fp32).
    """
    lib = load_library()
    _require_gpu(q, k, v)
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    if k.shape != (B, H, Sk, D) or v.shape != k.shape:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must share one dtype")
    _, nbytes = splitk_plan(q.dtype, B, H, Sq, Sk, D, num_splits)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    o, lse = _outputs(q, out, lse, (B, H, Sq))
    _check(lib.attn_fwd_splitk(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
        _dtype_code(q), B, H, Sq, Sk, D,
        _strides(q), _strides(k), _strides(v), _strides(o),
        _scale(scale, D), int(bool(causal)), int(num_splits), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream_handle(q.device)))
    return o, lse


def attn_fwd_splitk_noalloc(q, k, v, scale=None, causal=False, num_splits=0, out=None,
                            lse=None):
    """The split forward on the library's static per-device scratch (no
    workspace, nothing allocated by the library; calls that overlap on one
    GPU race).  Same arguments and results as attn_fwd_splitk without
    ``workspace``; a problem whose plan needs more than NOALLOC_SCRATCH_BYTES
    raises SdpaError (SDPA_ERR_SCRATCH).  Pass ``out`` and ``lse`` to
    allocate nothing here either."""
    lib = load_library()
    _require_gpu(q, k, v)
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    if k.shape != (B, H, Sk, D) or v.shape != k.shape:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must share one dtype")
    o, lse = _outputs(q, out, lse, (B, H, Sq))
    with torch.cuda.device(q.device):
        _check(lib.attn_fwd_splitk_noalloc(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
            _dtype_code(q), B, H, Sq, Sk, D,
            _strides(q), _strides(k), _strides(v), _strides(o),
            _scale(scale, D), int(bool(causal)), int(num_splits), _stream_handle(q.device)))
    return o, lse


def bwd_workspace_bytes(B: int, H: int, seqlen_q: int) -> int:
    """Workspace bytes attn_bwd needs for these sizes."""
    nbytes = ctypes.c_uint64()
    _check(load_library().sdpa_bwd_workspace_bytes(B, H, seqlen_q, ctypes.byref(nbytes)))
    return nbytes.value


def attn_bwd(q, k, v, o, dout, lse, scale=None, causal=False, dq=None, dk=None, dv=None,
             workspace=None):
    """Dense backward (bf16/fp16).  q: (B,H,Sq,D), k/v: (B,H,Sk,D), o/dout like q,
    lse (B,H,Sq) fp32 as attn_fwd returns them.  Returns (dq, dk, dv) shaped
    and strided like q, k, v (allocated with empty_like unless given)."""
    lib = load_library()
    _require_gpu(q, k, v, o, dout, lse)
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    if k.shape != (B, H, Sk, D) or v.shape != k.shape or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("shape mismatch among q, k, v, o, dout")
    if lse.shape != (B, H, Sq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous (B, H, Sq) float32 tensor")
    if len({t.dtype for t in (q, k, v, o, dout)}) != 1:
        raise ValueError("q, k, v, o and dout must share one dtype")
    dq, dk, dv = _grads_like(q, k, v, dq, dk, dv)
    if workspace is None:
        workspace = torch.empty(max(bwd_workspace_bytes(B, H, Sq), 1), dtype=torch.uint8,
                                device=q.device)
    _check(lib.attn_bwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), _dtype_code(q), B, H, Sq, Sk, D,
        _strides(q), _strides(k), _strides(v), _strides(o), _strides(dout),
        _scale(scale, D), int(bool(causal)), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream_handle(q.device)))
    return dq, dk, dv


def _device_cu(cu, device, total, max_len, check):
    if isinstance(cu, torch.Tensor) and cu.is_cuda:
        if cu.dtype != torch.int32:
            raise ValueError("cu_seqlens must be int32")
        return cu
    arr = np.asarray(cu.cpu().numpy() if isinstance(cu, torch.Tensor) else cu, dtype=np.int32)
    if check:
        check_cu_seqlens_host(arr, total, max_len)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


def _max_len(cu, given):
    if given is not None:
        return int(given)
    if isinstance(cu, torch.Tensor) and cu.is_cuda:
        raise ValueError("max_seqlen is required with device cu_seqlens")
    c = np.asarray(cu.cpu().numpy() if isinstance(cu, torch.Tensor) else cu, dtype=np.int64)
    return int(np.diff(c).max()) if c.size > 1 else 0


def _grads_like(q, k, v, dq, dk, dv):
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for g, t in ((dq, q), (dk, k), (dv, v)):
        if g.stride() != t.stride() or g.shape != t.shape or g.dtype != t.dtype:
            raise ValueError("dq, dk, dv must have the shapes, strides and dtype of q, k, v")
    return dq, dk, dv


def attn_fwd_compact_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q=None,
                            max_seqlen_k=None, scale=None, causal=False, out=None, lse=None,
                            check=True, bias=None):
    """Compact varlen forward over packed (T, H, D) tokens.

    cu_seqlens may be host arrays (checked with the library's host check,
    then copied to the device) or device int32 tensors (used as given).
    Returns (o (Tq,H,D), lse (1,H,Tq) fp32).  Max lengths default to the
    largest length in host cu_seqlens.  ``bias`` (optional) is broadcastable
    to (1, H, Tq, Tk); sequence z reads its block of it.
    """
    lib = load_library()
    _require_gpu(q, k, v)
    Tq, H, D = q.shape
    Tk = k.shape[0]
    if k.shape != (Tk, H, D) or v.shape != k.shape:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must share one dtype")

    max_q = _max_len(cu_seqlens_q, max_seqlen_q)
    max_k = _max_len(cu_seqlens_k, max_seqlen_k)
    cu_q = _device_cu(cu_seqlens_q, q.device, Tq, max_q, check)
    cu_k = _device_cu(cu_seqlens_k, q.device, Tk, max_k, check)
    if cu_q.numel() != cu_k.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k need the same length")
    num_seqs = cu_q.numel() - 1
    o, lse = _outputs(q, out, lse, (1, H, Tq))
    # (T, H, D) token memory seen as the rank-4 view (1, H, T, D).
    qv, kv, vv, ov = (t.transpose(0, 1).unsqueeze(0) for t in (q, k, v, o))
    if bias is None:
        _check(lib.attn_fwd_compact_varlen(
            qv.data_ptr(), kv.data_ptr(), vv.data_ptr(), ov.data_ptr(), lse.data_ptr(),
            _dtype_code(q), 1, H, Tq, Tk, D, cu_q.data_ptr(), cu_k.data_ptr(), num_seqs, max_q,
            max_k, _strides(qv), _strides(kv), _strides(vv), _strides(ov),
            _scale(scale, D), int(bool(causal)), _stream_handle(q.device)))
    else:
        bv = _bias_view(bias, q, (1, H, Tq, Tk))
        _check(lib.attn_fwd_compact_varlen_bias(
            qv.data_ptr(), kv.data_ptr(), vv.data_ptr(), bv.data_ptr(), ov.data_ptr(),
            lse.data_ptr(), _dtype_code(q), 1, H, Tq, Tk, D, cu_q.data_ptr(), cu_k.data_ptr(),
            num_seqs, max_q, max_k, _strides(qv), _strides(kv), _strides(vv), _strides(bv),
            _strides(ov), _scale(scale, D), int(bool(causal)), _stream_handle(q.device)))
    return o, lse


def attn_fwd_padded_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, scale=None, causal=False,
                           out=None, lse=None, check=True, bias=None):
    """Padded varlen forward.  q: (B,H,Sq_max,D), k/v: (B,H,Sk_max,D).

    Batch b's true lengths are the differences of cu_seqlens.  Rows past a
    true length are left as allocated (uninitialised unless ``out``/``lse``
    are given).  ``bias`` (optional) is broadcastable to
    (B, H, Sq_max, Sk_max).  Returns (o, lse (B,H,Sq_max) fp32).
    """
    lib = load_library()
    _require_gpu(q, k, v)
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    if k.shape != (B, H, Sk, D) or v.shape != k.shape:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must share one dtype")
    cu_q = _device_cu(cu_seqlens_q, q.device, B * Sq, Sq, check)
    cu_k = _device_cu(cu_seqlens_k, q.device, B * Sk, Sk, check)
    if cu_q.numel() != B + 1 or cu_k.numel() != B + 1:
        raise ValueError("padded varlen needs B + 1 cu_seqlens entries")
    o, lse = _outputs(q, out, lse, (B, H, Sq))
    if bias is None:
        _check(lib.attn_fwd_padded_varlen(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
            _dtype_code(q), B, H, Sq, Sk, D, cu_q.data_ptr(), cu_k.data_ptr(),
            _strides(q), _strides(k), _strides(v), _strides(o),
            _scale(scale, D), int(bool(causal)), _stream_handle(q.device)))
    else:
        bv = _bias_view(bias, q, (B, H, Sq, Sk))
        _check(lib.attn_fwd_padded_varlen_bias(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), bv.data_ptr(), o.data_ptr(), lse.data_ptr(),
            _dtype_code(q), B, H, Sq, Sk, D, cu_q.data_ptr(), cu_k.data_ptr(),
            _strides(q), _strides(k), _strides(v), _strides(bv), _strides(o),
            _scale(scale, D), int(bool(causal)), _stream_handle(q.device)))
    return o, lse


def attn_bwd_compact_varlen(q, k, v, o, dout, lse, cu_seqlens_q, cu_seqlens_k,
                            max_seqlen_q=None, max_seqlen_k=None, scale=None, causal=False,
                            dq=None, dk=None, dv=None, workspace=None, check=True):
    """Compact varlen backward over packed (T, H, D) tokens (bf16/fp16).

    o, dout: (Tq, H, D) like q; lse: (1, H, Tq) fp32 as
    attn_fwd_compact_varlen returns it.  cu_seqlens as for the forward.
    Returns (dq, dk, dv) shaped like q, k, v; tokens outside every sequence
    are left as allocated (uninitialised unless given).
    """
    lib = load_library()
    _require_gpu(q, k, v, o, dout, lse)
    Tq, H, D = q.shape
    Tk = k.shape[0]
    if k.shape != (Tk, H, D) or v.shape != k.shape or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("shape mismatch among q, k, v, o, dout")
    if lse.shape != (1, H, Tq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous (1, H, Tq) float32 tensor")
    if len({t.dtype for t in (q, k, v, o, dout)}) != 1:
        raise ValueError("q, k, v, o and dout must share one dtype")
    max_q = _max_len(cu_seqlens_q, max_seqlen_q)
    max_k = _max_len(cu_seqlens_k, max_seqlen_k)
    cu_q = _device_cu(cu_seqlens_q, q.device, Tq, max_q, check)
    cu_k = _device_cu(cu_seqlens_k, q.device, Tk, max_k, check)
    if cu_q.numel() != cu_k.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k need the same length")
    dq, dk, dv = _grads_like(q, k, v, dq, dk, dv)
    if workspace is None:
        workspace = torch.empty(max(bwd_workspace_bytes(1, H, Tq), 1), dtype=torch.uint8,
                                device=q.device)
    views = [t.transpose(0, 1).unsqueeze(0) for t in (q, k, v, o, dout, dq, dk, dv)]
    qv, kv, vv, ov, dov, dqv, dkv, dvv = views
    _check(lib.attn_bwd_compact_varlen(
        qv.data_ptr(), kv.data_ptr(), vv.data_ptr(), ov.data_ptr(), dov.data_ptr(),
        lse.data_ptr(), dqv.data_ptr(), dkv.data_ptr(), dvv.data_ptr(), _dtype_code(q), 1, H,
        Tq, Tk, D, cu_q.data_ptr(), cu_k.data_ptr(), cu_q.numel() - 1, max_q, max_k,
        _strides(qv), _strides(kv), _strides(vv), _strides(ov), _strides(dov),
        _scale(scale, D), int(bool(causal)), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream_handle(q.device)))
    return dq, dk, dv


def attn_bwd_padded_varlen(q, k, v, o, dout, lse, cu_seqlens_q, cu_seqlens_k, scale=None,
                           causal=False, dq=None, dk=None, dv=None, workspace=None, check=True):
    """Padded varlen backward (bf16/fp16).  q/o/dout: (B,H,Sq_max,D), k/v:
    (B,H,Sk_max,D), lse (B,H,Sq_max) fp32 as attn_fwd_padded_varlen returns
    it.  Returns (dq, dk, dv); rows past a batch's true length are left as
    allocated (uninitialised unless given)."""
    lib = load_library()
    _require_gpu(q, k, v, o, dout, lse)
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    if k.shape != (B, H, Sk, D) or v.shape != k.shape or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("shape mismatch among q, k, v, o, dout")
    if lse.shape != (B, H, Sq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous (B, H, Sq_max) float32 tensor")
    if len({t.dtype for t in (q, k, v, o, dout)}) != 1:
        raise ValueError("q, k, v, o and dout must share one dtype")
    cu_q = _device_cu(cu_seqlens_q, q.device, B * Sq, Sq, check)
    cu_k = _device_cu(cu_seqlens_k, q.device, B * Sk, Sk, check)
    if cu_q.numel() != B + 1 or cu_k.numel() != B + 1:
        raise ValueError("padded varlen needs B + 1 cu_seqlens entries")
    dq, dk, dv = _grads_like(q, k, v, dq, dk, dv)
    if workspace is None:
        workspace = torch.empty(max(bwd_workspace_bytes(B, H, Sq), 1), dtype=torch.uint8,
                                device=q.device)
    _check(lib.attn_bwd_padded_varlen(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), _dtype_code(q), B, H, Sq, Sk, D,
        cu_q.data_ptr(), cu_k.data_ptr(), _strides(q), _strides(k), _strides(v), _strides(o),
        _strides(dout), _scale(scale, D), int(bool(causal)), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream_handle(q.device)))
    return dq, dk, dv
