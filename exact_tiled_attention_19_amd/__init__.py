"""Fused exact-attention forward for AMD Instinct MI355X (gfx950).

``forward(q, k, v, ...)``, ``forward_fp8(q8, k8, v8, ...)``, ``forward_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, ...)`` and
``backward(q, k, v, o, lse, dout, ...)`` run the HIP kernels of ``libfa.so`` through its C ABI
(include/fa.h); PyTorch only supplies device memory and the stream.
"""

from .binding import (  # noqa: F401
    FA_ALIGN_BOTTOM_RIGHT,
    FA_ALIGN_TOP_LEFT,
    FA_DTYPE_BF16,
    FA_DTYPE_F32,
    FA_DTYPE_FP8_E4M3,
    FA_ERR_HIP,
    FA_ERR_INVALID_ARG,
    FA_ERR_SCRATCH_LIMIT,
    FA_ERR_UNSUPPORTED,
    FA_MASK_CAUSAL,
    FA_MASK_KEY_PADDING,
    FA_MASK_NONE,
    FA_OK,
    FaError,
    FaInvalidArgument,
    FaUnsupported,
    LIB_PATH,
    backward,
    fa_bwd,
    fa_fwd,
    fa_fwd_dropout,
    fa_fwd_fp8,
    fa_fwd_varlen,
    forward,
    forward_dropout,
    forward_fp8,
    forward_varlen,
    load_library,
    scratch_bytes,
    status_str,
    variant_count,
    varlen_workspace_size,
    version,
)
