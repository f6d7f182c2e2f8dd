"""Exact attention forward for AMD Instinct MI355X (gfx950): Python binding of libfa.

The work is done by the HIP kernels in ``libfa.so`` (built in-tree by
``io_aware_exact_23_amd.build``); this module only marshals arguments through ctypes. PyTorch
provides device memory and the stream. There is no fallback: if the library is missing, every
call raises ``FaError``.

Entry points mirror the C ABI in ``include/fa.h``:

* ``fa_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, kv_seqlens, stream)`` -- bf16
* ``fa_fwd_noalloc(...)`` -- bf16, the same arguments, allocates no device memory
* ``fa_fwd_f32(...)``                                                          -- fp32
* ``fa_fwd_window(q, k, v, o, lse, B, H, Nq, Nk, d, scale, window_left, window_right,
  kv_seqlens, stream)`` -- bf16, sliding-window mask
* ``fa_fwd_varlen(q, k, v, o, lse, B, H, total_q, total_k, max_seqlen_q, d, scale, window_left,
  window_right, cu_seqlens_q, cu_seqlens_k, stream)`` -- bf16, packed variable-length batch
* ``fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, Nq, Nk, d, scale, causal, kv_seqlens,
  stream)`` -- bf16 backward pass (gradients of fa_fwd)
* ``fa_std_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, kv_seqlens, workspace,
  workspace_bytes, stream)`` -- bf16, standard (materialising) algorithm, the baseline
* ``fa_std_workspace_bytes(B, H, Nq, Nk)``
* ``fa_quantize_fp8(x, y, descale, B, H, N, d, lens, transpose, stream)`` -- bf16 -> e4m3 with one
  scale per (b, h) slice, V optionally transposed
* ``fa_fp8_vt_cols(Nk)``
* ``fa_fwd_fp8(q8, k8, vt8, descale_q, descale_k, descale_v, o, lse, B, H, Nq, Nk, d, scale,
  causal, kv_seqlens, stream)`` -- e4m3 forward
* ``fa_status_string(status)``, ``fa_last_error()``, ``fa_build_info()``

Pointer arguments accept a torch tensor (its ``data_ptr()``), an int address or None; ``stream``
accepts a ``torch.cuda.Stream``, an int handle or None (the current torch stream).
``attention(q, k, v, ...)`` allocates O and lse with torch and calls the right entry point
(``window=(left, right)`` selects ``fa_fwd_window``); ``varlen_attention`` does the same for
packed sequences;
``standard_attention(q, k, v, ...)`` does the same for ``fa_std_fwd`` (bf16 only), allocating
its workspace with torch unless one is passed. ``quantize_fp8`` and ``attention_fp8`` allocate
the e4m3 tensors, scales and outputs for ``fa_quantize_fp8`` and ``fa_fwd_fp8``.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

__all__ = ["FaError", "fa_fwd", "fa_fwd_noalloc", "fa_fwd_f32", "fa_fwd_window", "fa_fwd_varlen", "fa_bwd",
           "attention_backward", "fa_std_fwd", "fa_quantize_fp8", "fa_fp8_vt_cols", "fa_fwd_fp8",
           "quantize_fp8", "attention_fp8",
           "fa_std_workspace_bytes", "fa_status_string", "fa_last_error", "fa_build_info", "attention",
           "varlen_attention", "standard_attention", "library_path", "load_library"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libfa.so")
_lib = None

FA_OK = 0
FA_ERR_INVALID_ARGUMENT = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_HIP = -3


class FaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libfa status {status}: {message}")
        self.status = status
        self.message = message


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libfa.so once; raise FaError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise FaError(FA_ERR_HIP, f"{_LIB_PATH} not found: build it with "
                                  "`python -m io_aware_exact_23_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, ci, cf = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    sig = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, cf, ci, vp, vp]
    for name in ("fa_fwd", "fa_fwd_f32", "fa_fwd_noalloc"):
        fn = getattr(lib, name)
        fn.argtypes = sig
        fn.restype = ci
    lib.fa_fwd_window.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, cf, ci, ci, vp, vp]
    lib.fa_fwd_window.restype = ci
    lib.fa_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, ci, ci, vp, vp, vp]
    lib.fa_fwd_varlen.restype = ci
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, cf, ci, vp, vp]
    lib.fa_bwd.restype = ci
    lib.fa_std_fwd.argtypes = sig[:13] + [vp, ctypes.c_size_t, vp]
    lib.fa_std_fwd.restype = ci
    lib.fa_std_workspace_bytes.argtypes = [ci, ci, ci, ci]
    lib.fa_std_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_quantize_fp8.argtypes = [vp, vp, vp, ci, ci, ci, ci, vp, ci, vp]
    lib.fa_quantize_fp8.restype = ci
    lib.fa_fp8_vt_cols.argtypes = [ci]
    lib.fa_fp8_vt_cols.restype = ci
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, cf, ci, vp, vp]
    lib.fa_fwd_fp8.restype = ci
    lib.fa_status_string.argtypes = [ci]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_last_error.argtypes = []
    lib.fa_last_error.restype = ctypes.c_char_p
    lib.fa_build_info.argtypes = []
    lib.fa_build_info.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return x.data_ptr() if x.numel() > 0 else None
    return int(x)


def _stream(s) -> Optional[int]:
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if hasattr(s, "cuda_stream"):
        return s.cuda_stream
    return int(s)


def fa_status_string(status: int) -> str:
    return load_library().fa_status_string(int(status)).decode()


def fa_last_error() -> str:
    return load_library().fa_last_error().decode()


def fa_build_info() -> str:
    return load_library().fa_build_info().decode()


def _call(name, q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, kv_seqlens, stream):
    lib = load_library()
    st = getattr(lib, name)(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H),
                            int(Nq), int(Nk), int(d), float(scale), int(causal),
                            _ptr(kv_seqlens), _stream(stream))
    if st != FA_OK:
        raise FaError(st, f"{fa_status_string(st)} ({fa_last_error()})")


def fa_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, kv_seqlens=None, stream=None) -> None:
    """bf16 forward; see include/fa.h for the contract."""
    _call("fa_fwd", q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, kv_seqlens, stream)


def fa_fwd_noalloc(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, kv_seqlens=None, stream=None) -> None:
    """bf16 forward that allocates no device memory (decode partials in the library's static
    scratch); see include/fa.h for the contract."""
    _call("fa_fwd_noalloc", q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, kv_seqlens, stream)


def fa_fwd_f32(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, kv_seqlens=None, stream=None) -> None:
    """fp32 forward; see include/fa.h for the contract."""
    _call("fa_fwd_f32", q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, kv_seqlens, stream)


def _raise(st):
    if st != FA_OK:
        raise FaError(st, f"{fa_status_string(st)} ({fa_last_error()})")


def fa_fwd_window(q, k, v, o, lse, B, H, Nq, Nk, d, scale, window_left, window_right,
                  kv_seqlens=None, stream=None) -> None:
    """bf16 forward with a sliding-window mask; see include/fa.h for the contract."""
    lib = load_library()
    _raise(lib.fa_fwd_window(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(Nq),
                             int(Nk), int(d), float(scale), int(window_left), int(window_right),
                             _ptr(kv_seqlens), _stream(stream)))


def fa_fwd_varlen(q, k, v, o, lse, B, H, total_q, total_k, max_seqlen_q, d, scale, window_left,
                  window_right, cu_seqlens_q, cu_seqlens_k, stream=None) -> None:
    """bf16 forward over a packed variable-length batch; see include/fa.h for the contract."""
    lib = load_library()
    _raise(lib.fa_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H),
                             int(total_q), int(total_k), int(max_seqlen_q), int(d), float(scale),
                             int(window_left), int(window_right), _ptr(cu_seqlens_q),
                             _ptr(cu_seqlens_k), _stream(stream)))


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, Nq, Nk, d, scale, causal, kv_seqlens=None,
           stream=None) -> None:
    """bf16 backward pass; see include/fa.h for the contract."""
    lib = load_library()
    _raise(lib.fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                      _ptr(dv), int(B), int(H), int(Nq), int(Nk), int(d), float(scale), int(causal),
                      _ptr(kv_seqlens), _stream(stream)))


def attention_backward(q, k, v, o, lse, dout, scale: Optional[float] = None, causal: bool = False,
                       kv_seqlens=None, stream=None):
    """dQ, dK, dV (bf16) of attention(q, k, v) for the upstream gradient dout, given the forward's
    o and lse."""
    import torch

    B, H, Nq, Nk, d = _check_qkv(q, k, v, kv_seqlens, (torch.bfloat16,))
    for t in (o, dout):
        if (t.dtype != torch.bfloat16 or tuple(t.shape) != (B, H, Nq, d) or not t.is_contiguous()
                or t.device != q.device):
            raise ValueError("o and dout must be contiguous bf16 [B, H, Nq, d] on q's device")
    if (lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, Nq) or not lse.is_contiguous()
            or lse.device != q.device):
        raise ValueError("lse must be the forward's contiguous float32 [B, H, Nq] on q's device")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, Nq, Nk, d, scale, int(bool(causal)), kv_seqlens,
           stream)
    return dq, dk, dv


def varlen_attention(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int,
                     scale: Optional[float] = None, window=(-1, -1), out=None, lse=None,
                     stream=None) -> Tuple["object", "object"]:
    """O [H, Tq, d] and lse [H, Tq] for packed bf16 q [H, Tq, d], k, v [H, Tk, d]."""
    import torch

    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be [H, T, d]")
    H, Tq, d = q.shape
    Tk = k.shape[1]
    if tuple(k.shape) != (H, Tk, d) or tuple(v.shape) != (H, Tk, d):
        raise ValueError("k and v must be [H, Tk, d] matching q")
    for t in (q, k, v):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous bfloat16 device tensors")
    for c in (cu_seqlens_q, cu_seqlens_k):
        if c.dtype != torch.int32 or not c.is_cuda or not c.is_contiguous():
            raise ValueError("cu_seqlens must be contiguous int32 device tensors")
    B = cu_seqlens_q.numel() - 1
    if B < 0 or cu_seqlens_k.numel() != B + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both have B + 1 entries")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, lse = _out_lse(out, lse, (H, Tq, d), q.dtype, (H, Tq), q.device)
    fa_fwd_varlen(q, k, v, out, lse, B, H, Tq, Tk, max_seqlen_q, d, scale, window[0], window[1],
                  cu_seqlens_q, cu_seqlens_k, stream)
    return out, lse


def fa_std_workspace_bytes(B, H, Nq, Nk) -> int:
    """Workspace bytes fa_std_fwd needs; see include/fa.h."""
    return int(load_library().fa_std_workspace_bytes(int(B), int(H), int(Nq), int(Nk)))


def fa_std_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, kv_seqlens, workspace,
               workspace_bytes, stream=None) -> None:
    """bf16 forward by the standard algorithm; see include/fa.h for the contract."""
    lib = load_library()
    st = lib.fa_std_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(Nq),
                        int(Nk), int(d), float(scale), int(causal), _ptr(kv_seqlens),
                        _ptr(workspace), int(workspace_bytes), _stream(stream))
    if st != FA_OK:
        raise FaError(st, f"{fa_status_string(st)} ({fa_last_error()})")


def _raise_on(st) -> None:
    if st != FA_OK:
        raise FaError(st, f"{fa_status_string(st)} ({fa_last_error()})")


def fa_quantize_fp8(x, y, descale, B, H, N, d, lens=None, transpose=0, stream=None) -> None:
    """bf16 -> e4m3 with one scale per (b, h) slice; see include/fa.h for the contract."""
    lib = load_library()
    _raise_on(lib.fa_quantize_fp8(_ptr(x), _ptr(y), _ptr(descale), int(B), int(H), int(N), int(d),
                                  _ptr(lens), int(transpose), _stream(stream)))


def fa_fp8_vt_cols(Nk) -> int:
    """Columns of a transposed e4m3 V (Nk rounded up to 64)."""
    return int(load_library().fa_fp8_vt_cols(int(Nk)))


def fa_fwd_fp8(q8, k8, vt8, descale_q, descale_k, descale_v, o, lse, B, H, Nq, Nk, d, scale, causal,
               kv_seqlens=None, stream=None) -> None:
    """e4m3 forward; see include/fa.h for the contract."""
    lib = load_library()
    _raise_on(lib.fa_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(vt8), _ptr(descale_q), _ptr(descale_k),
                             _ptr(descale_v), _ptr(o), _ptr(lse), int(B), int(H), int(Nq), int(Nk),
                             int(d), float(scale), int(causal), _ptr(kv_seqlens), _stream(stream)))


def quantize_fp8(x, kv_seqlens=None, transpose: bool = False, stream=None):
    """(codes, descale) for a contiguous bf16 device tensor x [B, H, N, d]: codes uint8
    [B, H, N, d], or [B, H, d, fa_fp8_vt_cols(N)] when transpose; descale fp32 [B, H]."""
    import torch

    if x.dim() != 4 or x.dtype != torch.bfloat16 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous bfloat16 device tensor [B, H, N, d]")
    B, H, N, d = x.shape
    if kv_seqlens is not None and (kv_seqlens.dtype != torch.int32 or not kv_seqlens.is_cuda
                                   or kv_seqlens.numel() != B or not kv_seqlens.is_contiguous()):
        raise ValueError("kv_seqlens must be a contiguous int32 device tensor of length B")
    shape = (B, H, d, fa_fp8_vt_cols(N)) if transpose else (B, H, N, d)
    y = torch.empty(shape, dtype=torch.uint8, device=x.device)
    descale = torch.empty((B, H), dtype=torch.float32, device=x.device)
    fa_quantize_fp8(x, y, descale, B, H, N, d, kv_seqlens, int(bool(transpose)), stream)
    return y, descale


def attention_fp8(q8, k8, vt8, descale_q, descale_k, descale_v, scale: Optional[float] = None,
                  causal: bool = False, kv_seqlens=None, out=None, lse=None,
                  stream=None) -> Tuple["object", "object"]:
    """O (bf16) and lse for e4m3 q8 [B,H,Nq,d], k8 [B,H,Nk,d], vt8 [B,H,d,fa_fp8_vt_cols(Nk)]."""
    import torch

    if q8.dim() != 4 or k8.dim() != 4 or vt8.dim() != 4:
        raise ValueError("q8, k8, vt8 must be 4-d")
    B, H, Nq, d = q8.shape
    Nk = k8.shape[2]
    if tuple(k8.shape) != (B, H, Nk, d) or tuple(vt8.shape) != (B, H, d, fa_fp8_vt_cols(Nk)):
        raise ValueError("k8 must be [B, H, Nk, d] and vt8 [B, H, d, fa_fp8_vt_cols(Nk)]")
    for t in (q8, k8, vt8):
        if t.dtype != torch.uint8 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("q8, k8, vt8 must be contiguous uint8 device tensors")
    for t in (descale_q, descale_k, descale_v):
        if t is not None and (t.dtype != torch.float32 or t.numel() != B * H or not t.is_cuda
                              or not t.is_contiguous()):
            raise ValueError("descales must be fp32 device tensors of B*H entries (or None)")
    if kv_seqlens is not None and (kv_seqlens.dtype != torch.int32 or not kv_seqlens.is_cuda
                                   or kv_seqlens.numel() != B or not kv_seqlens.is_contiguous()):
        raise ValueError("kv_seqlens must be a contiguous int32 device tensor of length B")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, lse = _out_lse(out, lse, (B, H, Nq, d), torch.bfloat16, (B, H, Nq), q8.device)
    fa_fwd_fp8(q8, k8, vt8, descale_q, descale_k, descale_v, out, lse, B, H, Nq, Nk, d, scale,
               int(bool(causal)), kv_seqlens, stream)
    return out, lse


def _out_lse(out, lse, o_shape, o_dtype, l_shape, device):
    """The caller's O and lse tensors, checked (the kernels write exactly these shapes, so a smaller
    or strided buffer would be written past its end), or new ones."""
    import torch

    if out is None:
        out = torch.empty(o_shape, dtype=o_dtype, device=device)
    elif (tuple(out.shape) != tuple(o_shape) or out.dtype != o_dtype or out.device != device
          or not out.is_contiguous()):
        raise ValueError(f"out must be a contiguous {o_dtype} tensor of shape {tuple(o_shape)} on {device}")
    if lse is None:
        lse = torch.empty(l_shape, dtype=torch.float32, device=device)
    elif (tuple(lse.shape) != tuple(l_shape) or lse.dtype != torch.float32 or lse.device != device
          or not lse.is_contiguous()):
        raise ValueError(f"lse must be a contiguous float32 tensor of shape {tuple(l_shape)} on {device}")
    return out, lse


def _check_qkv(q, k, v, kv_seqlens, dtypes):
    import torch

    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if tuple(k.shape) != (B, H, Nk, d) or tuple(v.shape) != (B, H, Nk, d):
        raise ValueError("k and v must be [B, H, Nk, d] matching q")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in dtypes:
        raise ValueError("q, k, v must share one of the dtypes " + ", ".join(map(str, dtypes)))
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous() or t.device != q.device:
            raise ValueError("q, k, v must be contiguous tensors on one device")
    if kv_seqlens is not None:
        if (kv_seqlens.dtype != torch.int32 or kv_seqlens.device != q.device or kv_seqlens.numel() != B
                or not kv_seqlens.is_contiguous()):
            raise ValueError("kv_seqlens must be a contiguous int32 tensor of length B on q's device")
    return B, H, Nq, Nk, d


def standard_attention(q, k, v, scale: Optional[float] = None, causal: bool = False,
                       kv_seqlens=None, out=None, lse=None, workspace=None,
                       stream=None) -> Tuple["object", "object"]:
    """O, lse by the standard algorithm (S and P through device memory), bf16 inputs."""
    import torch

    B, H, Nq, Nk, d = _check_qkv(q, k, v, kv_seqlens, (torch.bfloat16,))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, lse = _out_lse(out, lse, q.shape, q.dtype, (B, H, Nq), q.device)
    need = fa_std_workspace_bytes(B, H, Nq, Nk)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    fa_std_fwd(q, k, v, out, lse, B, H, Nq, Nk, d, scale, int(bool(causal)), kv_seqlens,
               workspace, wbytes, stream)
    return out, lse


def attention(q, k, v, scale: Optional[float] = None, causal: bool = False, kv_seqlens=None,
              out=None, lse=None, stream=None, window=None) -> Tuple["object", "object"]:
    """O, lse for device tensors q [B,H,Nq,d] and k, v [B,H,Nk,d] (bf16 or fp32, contiguous).

    window=(left, right) applies a sliding-window mask (bf16 only, not together with causal)."""
    import torch

    B, H, Nq, Nk, d = _check_qkv(q, k, v, kv_seqlens, (torch.bfloat16, torch.float32))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, lse = _out_lse(out, lse, q.shape, q.dtype, (B, H, Nq), q.device)
    if window is not None:
        if causal or q.dtype != torch.bfloat16:
            raise ValueError("window needs bf16 inputs and causal=False (use window (-1, 0))")
        fa_fwd_window(q, k, v, out, lse, B, H, Nq, Nk, d, scale, window[0], window[1], kv_seqlens,
                      stream)
        return out, lse
    fn = fa_fwd if q.dtype == torch.bfloat16 else fa_fwd_f32
    fn(q, k, v, out, lse, B, H, Nq, Nk, d, scale, int(bool(causal)), kv_seqlens, stream)
    return out, lse
