"""Seeded synthetic inputs for the attention forward workloads.

This module only draws and shapes random numbers; it holds none of the attention
arithmetic, so both the fp64 oracle and the HIP path can take their inputs from it
without sharing any of the method's code.

The five named workloads are the ones the attention-forward benchmark is quoted on.
The memory-budget exercise of "FlashAttention Interview Questions: IO Complexity,
Tiling, and Numerical Stability" (section "Which complexity becomes smaller, and
which does not?") uses N=4096, d=64 for one head, which is the ``c1`` workload.

Draw order for every workload (all from one ``torch.Generator('cpu')`` seeded with
the workload's seed): Q, K, V as float32 standard normals of shape [B, H, N, d];
then (key padding only) one valid key length per batch element, an integer uniform
on [N/2, N]; then (sampled-row checks only) for each (b, h) ``randperm(N)[:rows]``,
sorted.  Q and K are multiplied by ``qk_gain`` before the cast to the input dtype
(round to nearest even for bf16).
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

MASK_NONE = 0
MASK_CAUSAL = 1
MASK_KEY_PADDING = 2


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    in_dtype: torch.dtype
    out_dtypes: tuple
    mask_kinds: tuple          # each entry is a MASK_* bit set; the workload is run once per entry
    seed: int
    qk_gain: float = 1.0
    sample_rows: Optional[int] = None   # rows per head the oracle checks at full size (None = all)
    description: str = ""

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(d), as the float32 value the kernel receives."""
        return float(torch.tensor(1.0 / math.sqrt(self.d), dtype=torch.float32).item())


WORKLOADS = {
    "c0": Workload("c0", 1, 1, 256, 64, torch.float32, (torch.float32,), (MASK_NONE,), seed=0,
                   description="single head, fp32 inputs, no mask"),
    "c1": Workload("c1", 1, 1, 4096, 64, torch.bfloat16, (torch.bfloat16, torch.float32),
                   (MASK_NONE, MASK_CAUSAL), seed=1,
                   description="memory-budget example N=4096 d=64; non-causal and causal; bf16 and fp32 out"),
    "c2": Workload("c2", 4, 16, 8192, 128, torch.bfloat16, (torch.bfloat16,), (MASK_CAUSAL,), seed=2,
                   description="batched causal, the throughput/roofline workload"),
    "c3": Workload("c3", 2, 32, 16384, 64, torch.bfloat16, (torch.bfloat16,), (MASK_KEY_PADDING,), seed=3,
                   qk_gain=3.0, description="key padding, Q and K x3 so logit std ~ 9"),
    "c4": Workload("c4", 1, 8, 131072, 128, torch.bfloat16, (torch.bfloat16,), (MASK_CAUSAL,), seed=4,
                   sample_rows=1024, description="long-context causal, 1024 sampled rows per head"),
}


# Short-sequence bandwidth probes (not among the five named workloads): non-causal heads so
# short that the forward is bound by HBM traffic rather than by the MFMAs (arithmetic intensity
# N/2 FLOP per byte for bf16 in and out, below the ~315 FLOP/B ridge of the chip), with B*H
# chosen so that Q, K, V and O together take about 1 GiB.
PROBES = {
    f"bw{n}d{d}": Workload(f"bw{n}d{d}", (1 << 30) // (4 * n * d * 2) // 64, 64, n, d, torch.bfloat16,
                           (torch.bfloat16,), (MASK_NONE,), seed=10, sample_rows=64,
                           description=f"HBM-bound probe, N={n}, d={d}, Q+K+V+O = 1 GiB")
    for n in (128, 256, 512) for d in (64, 128)
}


@dataclasses.dataclass
class Inputs:
    q: torch.Tensor          # [B,H,N,d] CPU, in_dtype
    k: torch.Tensor
    v: torch.Tensor
    seqlens: Optional[torch.Tensor]   # [B] int32 CPU, or None
    rows: Optional[torch.Tensor]      # [B,H,R] int64 CPU sorted, or None
    scale: float


def random_qkv(B: int, H: int, N: int, d: int, dtype: torch.dtype, seed: int,
               qk_gain: float = 1.0):
    """Q, K, V standard normals (Q, K times ``qk_gain``) cast to ``dtype``; CPU tensors."""
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn(B, H, N, d, generator=g, dtype=torch.float32)
    k = torch.randn(B, H, N, d, generator=g, dtype=torch.float32)
    v = torch.randn(B, H, N, d, generator=g, dtype=torch.float32)
    if qk_gain != 1.0:
        q.mul_(qk_gain)
        k.mul_(qk_gain)
    return q.to(dtype), k.to(dtype), v.to(dtype), g


def ramp_qkv(B: int, H: int, N: int, d: int, span: float, dtype: torch.dtype, seed: int):
    """Logits that climb steadily along the keys: q_i = a u + 0.05 n_i, k_j = a (j / N) u + 0.05 n_j
    (u the all-ones vector, n standard normals), V standard normal, cast to ``dtype``; CPU tensors.

    a = sqrt(span / sqrt(d)), so with the scale 1/sqrt(d) the score of key j for any query is about
    span * j / N: each key tile raises the row maximum a little and the whole row climbs by about
    ``span`` (natural-log units).  Draw order: the query noise, the key noise, V.
    """
    g = torch.Generator("cpu").manual_seed(seed)
    a = math.sqrt(span / math.sqrt(d))
    ramp = torch.arange(N, dtype=torch.float32) / N
    q = a + 0.05 * torch.randn(B, H, N, d, generator=g, dtype=torch.float32)
    k = a * ramp[:, None] + 0.05 * torch.randn(B, H, N, d, generator=g, dtype=torch.float32)
    v = torch.randn(B, H, N, d, generator=g, dtype=torch.float32)
    return q.to(dtype), k.to(dtype), v.to(dtype)


def to_e4m3(x: torch.Tensor):
    """Per-tensor amax quantisation of a float tensor to FP8 E4M3 codes: (uint8 codes, descale).

    descale = max|x| / 448 (as float32; 1 for an all-zero tensor), codes = E4M3 of x / descale
    rounded to nearest even, clamped to +-448 first.  Input generation only: what the codes
    mean is fixed by the format, and both sides take them as given.
    """
    amax = float(x.abs().max()) if x.numel() else 0.0
    descale = float(torch.tensor(amax / 448.0 if amax > 0 else 1.0, dtype=torch.float32))
    y = (x.float() / descale).clamp(-448.0, 448.0)
    return y.to(torch.float8_e4m3fn).view(torch.uint8).contiguous(), descale


def random_qkv_fp8(B: int, H: int, N: int, d: int, seed: int, qk_gain: float = 1.0):
    """The normals of ``random_qkv`` (same seed, same draw order) quantised per tensor to E4M3:
    (q8, k8, v8, (descale_q, descale_k, descale_v)), uint8 CPU tensors."""
    q, k, v, _ = random_qkv(B, H, N, d, torch.float32, seed, qk_gain)
    (q8, dq), (k8, dk), (v8, dv) = to_e4m3(q), to_e4m3(k), to_e4m3(v)
    return q8, k8, v8, (dq, dk, dv)


def draw_seqlens(g: torch.Generator, B: int, N: int) -> torch.Tensor:
    """One valid key length per batch element, integer uniform on [N/2, N]."""
    return torch.randint(N // 2, N + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)


def draw_rows(g: torch.Generator, B: int, H: int, N: int, R: int) -> torch.Tensor:
    """For each (b, h), R distinct query rows chosen by ``randperm``, sorted."""
    out = torch.empty(B, H, min(R, N), dtype=torch.int64)
    for b in range(B):
        for h in range(H):
            out[b, h] = torch.sort(torch.randperm(N, generator=g)[:R]).values
    return out


def make_inputs(w: Workload, mask_kind: Optional[int] = None, sample_rows: Optional[int] = None) -> Inputs:
    """Inputs of workload ``w`` in the documented draw order."""
    q, k, v, g = random_qkv(w.B, w.H, w.N, w.d, w.in_dtype, w.seed, w.qk_gain)
    mk = w.mask_kinds[0] if mask_kind is None else mask_kind
    seqlens = draw_seqlens(g, w.B, w.N) if (mk & MASK_KEY_PADDING) else None
    R = w.sample_rows if sample_rows is None else sample_rows
    rows = draw_rows(g, w.B, w.H, w.N, R) if R is not None else None
    return Inputs(q, k, v, seqlens, rows, w.scale)


# ---- packed variable-length workloads --------------------------------------------------------
# The pages name decoding, unequal query/key lengths and packed sequences as cases whose key
# visibility must be settled explicitly, but quote no sizes for them; these stand-ins reuse the
# key/value shapes and token budgets of the named workloads above.
@dataclasses.dataclass(frozen=True)
class PackedWorkload:
    name: str
    H: int
    d: int
    lq: tuple                 # query length of every sequence
    lk: tuple                 # key length of every sequence
    causal: bool
    align: str                # "bottom_right" or "top_left"
    seed: int
    sample_seqs: Optional[int] = None   # sequences the oracle checks at full size (None = all)
    description: str = ""

    @property
    def scale(self) -> float:
        return scale_for(self.d)


def draw_lengths(seed: int, n: int, lo: int, hi: int) -> tuple:
    """n sequence lengths, integers uniform on [lo, hi], from their own generator."""
    g = torch.Generator("cpu").manual_seed(seed)
    return tuple(int(x) for x in torch.randint(lo, hi + 1, (n,), generator=g))


_MIX = draw_lengths(7, 16, 256, 4096)
PACKED = {
    "decode_c2kv": PackedWorkload("decode_c2kv", 16, 128, (1,) * 4, (8192,) * 4, True, "bottom_right", seed=20,
                                  description="one new query row per sequence against the c2 key/value shape "
                                              "(B=4, H=16, 8192 keys, d=128)"),
    "decode_c4kv": PackedWorkload("decode_c4kv", 8, 128, (1,), (131072,), True, "bottom_right", seed=21,
                                  description="one new query row against the c4 key/value shape "
                                              "(H=8, 131072 keys, d=128)"),
    "chunked_prefill": PackedWorkload("chunked_prefill", 16, 128, (512,) * 4, (8192,) * 4, True, "bottom_right",
                                      seed=22, sample_seqs=1,
                                      description="the last 512 positions of four 8192-token sequences "
                                                  "(H=16, d=128), bottom-right causal"),
    "single_4k_d64": PackedWorkload("single_4k_d64", 1, 64, (4096,), (4096,), False, "bottom_right", seed=24,
                                    sample_seqs=1,
                                    description="one 4096-token sequence, H=1, d=64, no mask (the c1 shape) through "
                                                "the packed entry point, whose workspace lets the keys split across "
                                                "workgroups"),
    "single_8k_d128": PackedWorkload("single_8k_d128", 2, 128, (8192,), (8192,), True, "bottom_right", seed=25,
                                     sample_seqs=1,
                                     description="one 8192-token causal sequence, H=2, d=128, through the packed "
                                                 "entry point"),
    "varlen_mix": PackedWorkload("varlen_mix", 16, 128, _MIX, _MIX, True, "bottom_right", seed=23, sample_seqs=2,
                                 description="16 packed causal sequences, lengths uniform on [256, 4096] "
                                             f"({sum(_MIX)} tokens, H=16, d=128)"),
}


def random_packed(lq, lk, H: int, d: int, dtype: torch.dtype, seed: int, qk_gain: float = 1.0):
    """Token-major packed inputs: Q [sum(lq), H, d], K and V [sum(lk), H, d] (standard normals,
    Q and K times ``qk_gain``, cast to ``dtype``) and the int32 prefix sums of the lengths."""
    g = torch.Generator("cpu").manual_seed(seed)
    Tq, Tk = int(sum(lq)), int(sum(lk))
    q = torch.randn(Tq, H, d, generator=g, dtype=torch.float32)
    k = torch.randn(Tk, H, d, generator=g, dtype=torch.float32)
    v = torch.randn(Tk, H, d, generator=g, dtype=torch.float32)
    if qk_gain != 1.0:
        q.mul_(qk_gain)
        k.mul_(qk_gain)
    cu_q = torch.tensor([0] + [int(x) for x in torch.cumsum(torch.tensor(lq, dtype=torch.int64), 0)], dtype=torch.int32)
    cu_k = torch.tensor([0] + [int(x) for x in torch.cumsum(torch.tensor(lk, dtype=torch.int64), 0)], dtype=torch.int32)
    return q.to(dtype), k.to(dtype), v.to(dtype), cu_q, cu_k


def scale_for(d: int) -> float:
    """1/sqrt(d) rounded to float32, the value passed across the C ABI."""
    return float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32).item())
