"""fp64 CPU oracle for attention on 8-bit floating-point inputs -- TEST INFRASTRUCTURE.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import this
module.  It shares no code with the HIP path and imports nothing from it.

Source: "FlashAttention 1, 2 & 3: Memory Tiling & Eliminating the O(N^2) HBM Bottleneck"
(learn-interview-questions, Q18), section 3 (the table of kernel generations), names FP8
support as one of the hardware features the third generation exploits.  The pages fix
nothing else about it.  Readings (each also listed in the design notes):

* The 8-bit format is OCP FP8 E4M3 (the "fn" variant): one sign bit, four exponent bits
  with bias 7, three mantissa bits.  Exponent field 0 holds the subnormals m * 2^-9; the
  two codes with every exponent and mantissa bit set (0x7F, 0xFF) are NaN; there are no
  infinities, so the largest finite magnitude is 1.75 * 2^8 = 448.
* Each of Q, K and V carries one float32 descale factor per tensor: the real input is
  descale * decoded code.  Quantising a float tensor into codes is the caller's business.
* The attention itself is the plain definition on those real inputs, exactly as for bf16
  inputs (section "What is FlashAttention exact about?" of "FlashAttention Interview
  Questions: IO Complexity, Tiling, and Numerical Stability"), so after decoding this
  oracle hands the exact float64 values to ``attention_ref``.  Decoded codes have at most
  four significant bits and the descales 24, so every product is exact in float64.

Pinned by: the OCP format's fixed points (0x38 = 1, 0x7E = 448, 0x08 = 2^-6, 0x01 = 2^-9,
NaN codes, signed zero), agreement of all 256 codes with PyTorch's float8_e4m3fn decoding
(a library routine), monotonicity, the pages' two-key worked example carried in 8-bit
codes with a descale, and descale invariances (tests/oracle_fp8_pins.py).
"""

from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .attention import attention_ref


def e4m3_decode(codes) -> np.ndarray:
    """float64 values of OCP FP8 E4M3 codes (uint8 array or anything convertible to one).

    value = (-1)^s * 2^(e - 7) * (1 + m/8)  for exponent field e in 1..15,
            (-1)^s * 2^-6 * (m/8)           for e = 0 (subnormal),
    and NaN for the codes 0x7F and 0xFF.
    """
    if hasattr(codes, "detach"):
        codes = codes.detach().cpu().numpy()
    c = np.asarray(codes)
    if c.dtype != np.uint8:
        c = c.view(np.uint8) if c.dtype.itemsize == 1 else c.astype(np.uint8)
    c = c.astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    sub = np.ldexp(m / 8.0, -6)
    mag = np.where(e == 0, sub, normal)
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def dequantize(codes, descale: float) -> np.ndarray:
    """descale * decoded codes, in float64 (descale is taken as the float32 the kernel gets)."""
    return np.float64(np.float32(descale)) * e4m3_decode(codes)


def attention_fp8_ref(q8, k8, v8, descale_q: float, descale_k: float, descale_v: float, scale: float,
                      causal: bool = False, seqlens: Optional[Sequence[int]] = None, rows=None):
    """Exact attention of the dequantised 8-bit inputs ([B, H, N, d] codes): (O, LSE) in float64.

    O = softmax(scale * Qr Kr^T with masked keys removed) Vr with Qr = descale_q * Q8 etc.; the
    masks, the empty-row convention and ``rows`` are those of ``attention_ref``.
    """
    q = dequantize(q8, descale_q)
    k = dequantize(k8, descale_k)
    v = dequantize(v8, descale_v)
    return attention_ref(q, k, v, scale, causal=causal, seqlens=seqlens, rows=rows)
