"""Thin ctypes binding of ``libfa.so`` (the C ABI in include/fa.h).

Argument marshalling only: PyTorch provides device memory and the current HIP stream; every
step of the attention forward runs in the library's HIP kernels.  There is no fallback: if
the library is missing or cannot be loaded, every call raises.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libfa.so")

FA_OK = 0
FA_ERR_INVALID_ARG = 1
FA_ERR_UNSUPPORTED = 2
FA_ERR_HIP = 3
FA_ERR_SCRATCH_LIMIT = 4

FA_MASK_NONE = 0
FA_MASK_CAUSAL = 1
FA_MASK_KEY_PADDING = 2

FA_DTYPE_F32 = 0
FA_DTYPE_BF16 = 1
FA_DTYPE_FP8_E4M3 = 2

FA_ALIGN_BOTTOM_RIGHT = 0
FA_ALIGN_TOP_LEFT = 1
_ALIGN_CODE = {"bottom_right": FA_ALIGN_BOTTOM_RIGHT, "top_left": FA_ALIGN_TOP_LEFT}

_DTYPE_CODE = {torch.float32: FA_DTYPE_F32, torch.bfloat16: FA_DTYPE_BF16}

# Every symbol include/fa.h declares, with its ctypes signature.
_VP = ctypes.c_void_p
_I = ctypes.c_int
SIGNATURES = {
    "fa_fwd": (_I, [_VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, ctypes.c_float, _I, _VP, _I, _I, _VP]),
    "fa_fwd_fp8": (_I, [_VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                        ctypes.c_float, _I, _VP, _I, _VP]),
    "fa_fwd_variant": (_I, [_VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, ctypes.c_float, _I, _VP, _I, _I, _VP, _I]),
    "fa_fwd_dropout": (_I, [_VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, ctypes.c_float, _I, _VP, ctypes.c_float,
                            ctypes.c_uint64, ctypes.c_uint32, _I, _I, _VP]),
    "fa_bwd": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, ctypes.c_float, _I, _VP, _I, _I,
                    _VP]),
    "fa_fwd_varlen": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _I, ctypes.c_float, _I, _I,
                           _VP, ctypes.c_size_t, _I, _I, _VP]),
    "fa_fwd_varlen_workspace_size": (ctypes.c_size_t, [_I, _I, _I, _I, _I]),
    "fa_fwd_varlen_noalloc": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _I, ctypes.c_float, _I,
                                   _I, _I, _I, _VP]),
    "fa_scratch_bytes": (ctypes.c_size_t, []),
    "fa_bwd_dropout": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, ctypes.c_float, _I, _VP,
                            ctypes.c_float, ctypes.c_uint64, ctypes.c_uint32, _I, _I, _VP]),
    "fa_variant_count": (_I, []),
    "fa_status_str": (ctypes.c_char_p, [_I]),
    "fa_last_hip_error": (_I, []),
    "fa_version": (_I, []),
}

_lib = None


class FaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class FaInvalidArgument(FaError, ValueError):
    pass


class FaUnsupported(FaError, ValueError):
    pass


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load (once) and return the HIP library; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m exact_tiled_attention_19_amd.build_lib` (needs hipcc)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load_library().fa_status_str(status).decode()


def _check(status: int) -> None:
    if status == FA_OK:
        return
    lib = load_library()
    msg = lib.fa_status_str(status).decode()
    if status == FA_ERR_INVALID_ARG:
        raise FaInvalidArgument(status, msg)
    if status == FA_ERR_UNSUPPORTED:
        raise FaUnsupported(status, msg)
    if status == FA_ERR_HIP:
        raise FaError(status, f"{msg}: hipError_t {lib.fa_last_hip_error()}")
    raise FaError(status, msg)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def fa_fwd(q, k, v, o, lse, B, H, N, d, scale, mask_kind, seqlens, in_dtype, out_dtype, stream,
           variant: int = 0) -> int:
    """Raw call through the C ABI (pointers as ints or None); returns the status code."""
    lib = load_library()
    if variant == 0:
        return lib.fa_fwd(q, k, v, o, lse, B, H, N, d, ctypes.c_float(scale), mask_kind, seqlens,
                          in_dtype, out_dtype, stream)
    return lib.fa_fwd_variant(q, k, v, o, lse, B, H, N, d, ctypes.c_float(scale), mask_kind, seqlens,
                              in_dtype, out_dtype, stream, variant)


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, scale: Optional[float] = None,
            causal: bool = False, seqlens: Optional[torch.Tensor] = None,
            out_dtype: Optional[torch.dtype] = None, return_lse: bool = True,
            out: Optional[torch.Tensor] = None, lse_out: Optional[torch.Tensor] = None,
            variant: int = 0) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Exact attention forward on the GPU: returns (O, LSE).

    q, k, v: [B, H, N, d] contiguous device tensors of one dtype (bfloat16 or float32).
    scale: multiplier of q.k (default 1/sqrt(d), rounded to float32).
    causal: key j visible to query i only when j <= i.
    seqlens: optional int32 device tensor [B]; keys j >= seqlens[b] are masked.
    out_dtype: output dtype (default: the input dtype).
    out / lse_out: optional preallocated outputs.
    """
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be device tensors")
    if q.dtype != k.dtype or q.dtype != v.dtype or q.dtype not in _DTYPE_CODE:
        raise ValueError("q, k, v must share a dtype in {bfloat16, float32}")
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must all be [B, H, N, d]")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out_dtype not in _DTYPE_CODE:
        raise ValueError("out_dtype must be bfloat16 or float32")
    mask = FA_MASK_CAUSAL if causal else FA_MASK_NONE
    if seqlens is not None:
        if not seqlens.is_cuda or seqlens.dtype != torch.int32 or seqlens.numel() != B or not seqlens.is_contiguous():
            raise ValueError("seqlens must be a contiguous int32 device tensor with B entries")
        mask |= FA_MASK_KEY_PADDING
    if out is None:
        out = torch.empty((B, H, N, d), dtype=out_dtype, device=q.device)
    elif out.shape != q.shape or out.dtype != out_dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out has the wrong shape, dtype, layout or device")
    lse = None
    if return_lse:
        if lse_out is None:
            lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        else:
            if lse_out.shape != (B, H, N) or lse_out.dtype != torch.float32 or not lse_out.is_contiguous():
                raise ValueError("lse_out must be a contiguous float32 [B, H, N] tensor")
            lse = lse_out
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d, float(scale), mask,
                _ptr(seqlens), _DTYPE_CODE[q.dtype], _DTYPE_CODE[out_dtype], stream, variant)
    _check(st)
    return out, lse


def fa_fwd_fp8(q, k, v, o, lse, B, H, N, d, scale, descale_q, descale_k, descale_v, mask_kind, seqlens, out_dtype,
               stream) -> int:
    """Raw call of the 8-bit-input forward through the C ABI (pointers as ints or None)."""
    f = ctypes.c_float
    return load_library().fa_fwd_fp8(q, k, v, o, lse, B, H, N, d, f(scale), f(descale_q), f(descale_k), f(descale_v),
                                     mask_kind, seqlens, out_dtype, stream)


_FP8_DTYPES = (torch.uint8, torch.float8_e4m3fn)


def forward_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, descale_q: float = 1.0,
                descale_k: float = 1.0, descale_v: float = 1.0, scale: Optional[float] = None,
                causal: bool = False, seqlens: Optional[torch.Tensor] = None,
                out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None,
                lse_out: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Attention forward on FP8 E4M3 inputs (contract in include/fa.h): returns (O, LSE).

    q, k, v: [B, H, N, d] contiguous device tensors of E4M3 codes (torch.uint8 or
    torch.float8_e4m3fn); the real inputs are descale_* times the decoded codes.
    """
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be device tensors")
    if any(t.dtype not in _FP8_DTYPES for t in (q, k, v)):
        raise ValueError("q, k, v must hold E4M3 codes (uint8 or float8_e4m3fn)")
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape or not all(t.is_contiguous() for t in (q, k, v)):
        raise ValueError("q, k, v must all be contiguous [B, H, N, d]")
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if out_dtype not in _DTYPE_CODE:
        raise ValueError("out_dtype must be bfloat16 or float32")
    mask = FA_MASK_CAUSAL if causal else FA_MASK_NONE
    if seqlens is not None:
        if not seqlens.is_cuda or seqlens.dtype != torch.int32 or seqlens.numel() != B or not seqlens.is_contiguous():
            raise ValueError("seqlens must be a contiguous int32 device tensor with B entries")
        mask |= FA_MASK_KEY_PADDING
    if out is None:
        out = torch.empty((B, H, N, d), dtype=out_dtype, device=q.device)
    elif out.shape != q.shape or out.dtype != out_dtype or not out.is_contiguous():
        raise ValueError("out has the wrong shape, dtype or layout")
    if lse_out is None:
        lse_out = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    elif lse_out.shape != (B, H, N) or lse_out.dtype != torch.float32 or not lse_out.is_contiguous():
        raise ValueError("lse_out must be a contiguous float32 [B, H, N] tensor")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = fa_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse_out), B, H, N, d, float(scale), float(descale_q),
                    float(descale_k), float(descale_v), mask, _ptr(seqlens), _DTYPE_CODE[out_dtype], stream)
    _check(st)
    return out, lse_out


def fa_fwd_dropout(q, k, v, o, lse, B, H, N, d, scale, mask_kind, seqlens, p_drop, seed, offset, in_dtype, out_dtype,
                   stream) -> int:
    """Raw call of the forward with dropout through the C ABI (pointers as ints or None)."""
    return load_library().fa_fwd_dropout(q, k, v, o, lse, B, H, N, d, ctypes.c_float(scale), mask_kind, seqlens,
                                         ctypes.c_float(p_drop), ctypes.c_uint64(seed), ctypes.c_uint32(offset),
                                         in_dtype, out_dtype, stream)


def forward_dropout(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, p: float, seed: int, offset: int = 0, *,
                    scale: Optional[float] = None, causal: bool = False, seqlens: Optional[torch.Tensor] = None,
                    out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
                    lse_out: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Attention forward with dropout on the probabilities (contract in include/fa.h): returns
    (O, LSE), LSE before dropout.  q, k, v: [B, H, N, d] contiguous bfloat16 device tensors;
    p: drop probability (quantised to 1/256); seed (64-bit) and offset (32-bit) select the mask."""
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be device tensors")
    if q.dtype != torch.bfloat16 or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must be bfloat16")
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape or not all(t.is_contiguous() for t in (q, k, v)):
        raise ValueError("q, k, v must all be contiguous [B, H, N, d]")
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    if out_dtype not in _DTYPE_CODE:
        raise ValueError("out_dtype must be bfloat16 or float32")
    mask = FA_MASK_CAUSAL if causal else FA_MASK_NONE
    if seqlens is not None:
        if not seqlens.is_cuda or seqlens.dtype != torch.int32 or seqlens.numel() != B or not seqlens.is_contiguous():
            raise ValueError("seqlens must be a contiguous int32 device tensor with B entries")
        mask |= FA_MASK_KEY_PADDING
    if out is None:
        out = torch.empty((B, H, N, d), dtype=out_dtype, device=q.device)
    elif out.shape != q.shape or out.dtype != out_dtype or not out.is_contiguous():
        raise ValueError("out has the wrong shape, dtype or layout")
    if lse_out is None:
        lse_out = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    elif lse_out.shape != (B, H, N) or lse_out.dtype != torch.float32 or not lse_out.is_contiguous():
        raise ValueError("lse_out must be a contiguous float32 [B, H, N] tensor")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = fa_fwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse_out), B, H, N, d, float(scale), mask,
                        _ptr(seqlens), float(p), int(seed) & 0xFFFFFFFFFFFFFFFF, int(offset) & 0xFFFFFFFF,
                        FA_DTYPE_BF16, _DTYPE_CODE[out_dtype], stream)
    _check(st)
    return out, lse_out


def fa_bwd(q, k, v, o, lse, dout, delta, dq, dk, dv, B, H, N, d, scale, mask_kind, seqlens, in_dtype,
           grad_dtype, stream) -> int:
    """Raw call of the backward pass through the C ABI (pointers as ints or None)."""
    return load_library().fa_bwd(q, k, v, o, lse, dout, delta, dq, dk, dv, B, H, N, d, ctypes.c_float(scale),
                                 mask_kind, seqlens, in_dtype, grad_dtype, stream)


def backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
             dout: torch.Tensor, *, scale: Optional[float] = None, causal: bool = False,
             seqlens: Optional[torch.Tensor] = None, out: Optional[Tuple[torch.Tensor, ...]] = None,
             delta: Optional[torch.Tensor] = None,
             dropout: Optional[Tuple[float, int, int]] = None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Gradients (dQ, dK, dV) of the forward pass on the GPU, float32.

    q, k, v: the forward inputs; o, lse: what ``forward`` returned for them (o in bfloat16);
    dout: the gradient arriving at o.  All [B, H, N, d] contiguous bfloat16 device tensors (lse
    float32 [B, H, N]).  scale, causal and seqlens as for ``forward``.
    out: optional preallocated (dq, dk, dv) float32 tensors; delta: optional float32 [B, H, N]
    workspace (allocated here when omitted).  dropout: (p, seed, offset) of the
    ``forward_dropout`` call that produced o and lse, whose mask is regenerated.
    """
    ts = (q, k, v, o, dout)
    if not all(t.is_cuda for t in ts) or not lse.is_cuda:
        raise ValueError("all tensors must be device tensors")
    if any(t.dtype != torch.bfloat16 for t in ts):
        raise ValueError("q, k, v, o and dout must be bfloat16")
    if q.dim() != 4 or any(t.shape != q.shape for t in ts):
        raise ValueError("q, k, v, o and dout must all be [B, H, N, d]")
    if not all(t.is_contiguous() for t in ts):
        raise ValueError("q, k, v, o and dout must be contiguous")
    B, H, N, d = q.shape
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    mask = FA_MASK_CAUSAL if causal else FA_MASK_NONE
    if seqlens is not None:
        if not seqlens.is_cuda or seqlens.dtype != torch.int32 or seqlens.numel() != B or not seqlens.is_contiguous():
            raise ValueError("seqlens must be a contiguous int32 device tensor with B entries")
        mask |= FA_MASK_KEY_PADDING
    if out is None:
        out = tuple(torch.empty((B, H, N, d), dtype=torch.float32, device=q.device) for _ in range(3))
    elif len(out) != 3 or any(t.shape != q.shape or t.dtype != torch.float32 or not t.is_contiguous() for t in out):
        raise ValueError("out must be three contiguous float32 [B, H, N, d] tensors")
    if delta is None:
        delta = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    elif delta.shape != (B, H, N) or delta.dtype != torch.float32 or not delta.is_contiguous():
        raise ValueError("delta must be a contiguous float32 [B, H, N] tensor")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    if dropout is not None:
        p, seed, offset = dropout
        st = load_library().fa_bwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(delta),
                                           _ptr(out[0]), _ptr(out[1]), _ptr(out[2]), B, H, N, d, ctypes.c_float(scale),
                                           mask, _ptr(seqlens), ctypes.c_float(p),
                                           ctypes.c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF),
                                           ctypes.c_uint32(int(offset) & 0xFFFFFFFF), FA_DTYPE_BF16, FA_DTYPE_F32,
                                           stream)
        _check(st)
        return out
    st = fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(delta), _ptr(out[0]), _ptr(out[1]),
                _ptr(out[2]), B, H, N, d, float(scale), mask, _ptr(seqlens), FA_DTYPE_BF16, FA_DTYPE_F32, stream)
    _check(st)
    return out


def fa_fwd_varlen(q, k, v, o, lse, cu_q, cu_k, B, H, total_q, total_k, max_q, max_k, d, scale, mask_kind,
                  causal_align, workspace, workspace_bytes, in_dtype, out_dtype, stream) -> int:
    """Raw call of the packed variable-length forward through the C ABI (pointers as ints or None)."""
    return load_library().fa_fwd_varlen(q, k, v, o, lse, cu_q, cu_k, B, H, total_q, total_k, max_q, max_k, d,
                                        ctypes.c_float(scale), mask_kind, causal_align, workspace, workspace_bytes,
                                        in_dtype, out_dtype, stream)


def fa_fwd_varlen_noalloc(q, k, v, o, lse, cu_q, cu_k, B, H, total_q, total_k, max_q, max_k, d, scale, mask_kind,
                          causal_align, in_dtype, out_dtype, stream) -> int:
    """Raw call of the allocation-free packed forward through the C ABI (pointers as ints or None)."""
    return load_library().fa_fwd_varlen_noalloc(q, k, v, o, lse, cu_q, cu_k, B, H, total_q, total_k, max_q, max_k,
                                                d, ctypes.c_float(scale), mask_kind, causal_align, in_dtype,
                                                out_dtype, stream)


def scratch_bytes() -> int:
    return int(load_library().fa_scratch_bytes())


def varlen_workspace_size(B: int, H: int, max_seqlen_q: int, max_seqlen_k: int, d: int) -> int:
    return int(load_library().fa_fwd_varlen_workspace_size(B, H, max_seqlen_q, max_seqlen_k, d))


def forward_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
                   cu_seqlens_k: torch.Tensor, max_seqlen_q: Optional[int] = None,
                   max_seqlen_k: Optional[int] = None, *, scale: Optional[float] = None, causal: bool = False,
                   align: str = "bottom_right", out_dtype: Optional[torch.dtype] = None, return_lse: bool = True,
                   out: Optional[torch.Tensor] = None, lse_out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None,
                   noalloc: bool = False) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Exact attention over a packed batch of sequences on the GPU: returns (O, LSE).

    q: [Tq, H, d], k, v: [Tk, H, d] contiguous bfloat16 device tensors (token-major).
    cu_seqlens_q, cu_seqlens_k: contiguous int32 device tensors [B + 1], prefix sums of the
    per-sequence query and key lengths.  max_seqlen_q / max_seqlen_k: the longest lengths (read
    from the prefix sums, with a device synchronisation, when omitted).
    causal: key j visible to query row i iff j <= i + delta, delta = Lk - Lq for
    align="bottom_right" and 0 for align="top_left".
    Returns O [Tq, H, d] (out_dtype, default bfloat16) and LSE [H, Tq] float32.
    workspace: optional uint8 device tensor of at least ``varlen_workspace_size(...)`` bytes.
    noalloc: call fa_fwd_varlen_noalloc instead, whose workspace is the library's fixed device
    array (no workspace is allocated or passed; pass ``out`` and ``lse_out`` to allocate nothing).
    """
    ts = (q, k, v, cu_seqlens_q, cu_seqlens_k)
    if not all(t.is_cuda for t in ts):
        raise ValueError("all tensors must be device tensors")
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise ValueError("q, k, v must be bfloat16")
    if q.dim() != 3 or k.dim() != 3 or k.shape != v.shape or q.shape[1:] != k.shape[1:]:
        raise ValueError("q must be [Tq, H, d] and k, v [Tk, H, d]")
    if not all(t.is_contiguous() for t in ts):
        raise ValueError("all tensors must be contiguous")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32 or cu_seqlens_q.dim() != 1 \
            or cu_seqlens_q.shape != cu_seqlens_k.shape or cu_seqlens_q.numel() < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must be int32 [B + 1] tensors")
    if align not in _ALIGN_CODE:
        raise ValueError(f"align must be one of {sorted(_ALIGN_CODE)}")
    Tq, H, d = q.shape
    Tk = k.shape[0]
    B = cu_seqlens_q.numel() - 1
    if max_seqlen_q is None:
        max_seqlen_q = int((cu_seqlens_q[1:] - cu_seqlens_q[:-1]).max().item()) if B > 0 else 0
    if max_seqlen_k is None:
        max_seqlen_k = int((cu_seqlens_k[1:] - cu_seqlens_k[:-1]).max().item()) if B > 0 else 0
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    if out_dtype not in _DTYPE_CODE:
        raise ValueError("out_dtype must be bfloat16 or float32")
    if out is None:
        out = torch.empty((Tq, H, d), dtype=out_dtype, device=q.device)
    elif out.shape != q.shape or out.dtype != out_dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out has the wrong shape, dtype, layout or device")
    lse = None
    if return_lse:
        if lse_out is None:
            lse = torch.empty((H, Tq), dtype=torch.float32, device=q.device)
        else:
            if lse_out.shape != (H, Tq) or lse_out.dtype != torch.float32 or not lse_out.is_contiguous():
                raise ValueError("lse_out must be a contiguous float32 [H, Tq] tensor")
            lse = lse_out
    stream = torch.cuda.current_stream(q.device).cuda_stream
    if noalloc:
        if workspace is not None:
            raise ValueError("noalloc takes no workspace")
        st = fa_fwd_varlen_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens_q),
                                   _ptr(cu_seqlens_k), B, H, Tq, Tk, int(max_seqlen_q), int(max_seqlen_k), d,
                                   float(scale), FA_MASK_CAUSAL if causal else FA_MASK_NONE, _ALIGN_CODE[align],
                                   FA_DTYPE_BF16, _DTYPE_CODE[out_dtype], stream)
        _check(st)
        return out, lse
    ws_bytes = varlen_workspace_size(B, H, max_seqlen_q, max_seqlen_k, d)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_given = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = fa_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), B, H,
                       Tq, Tk, int(max_seqlen_q), int(max_seqlen_k), d, float(scale),
                       FA_MASK_CAUSAL if causal else FA_MASK_NONE, _ALIGN_CODE[align], _ptr(workspace), ws_given,
                       FA_DTYPE_BF16, _DTYPE_CODE[out_dtype], stream)
    _check(st)
    return out, lse


def variant_count() -> int:
    return load_library().fa_variant_count()


def version() -> int:
    return load_library().fa_version()
