"""Shared helpers of the GPU parity tests: run the HIP path, run the oracle, compare.

Tolerances (bf16 operands, float32 accumulation):
* float32 output: max |O - O_ref| <= 2e-4 and max |LSE - LSE_ref| <= 1e-4.
* bf16 output: every element within max(1e-2, half a bf16 ulp of O_ref + 1e-3).  Rounding
  the exact result to bf16 alone costs up to half an ulp, which exceeds 1e-2 once |O| >= 4
  (ulp 2^-5 on [4, 8)); below 4 the bound is exactly 1e-2.  LSE (float32) <= 1e-4.
* float32 inputs and output: the float32-output bounds.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import threadpoolctl
import torch

import exact_tiled_attention_19_amd as fa
import oracle

TOL_O_F32 = 2e-4
TOL_LSE = 1e-4
TOL_O_BF16 = 1e-2


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def bf16_bound(ref: np.ndarray) -> np.ndarray:
    a = np.abs(ref)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    half_ulp = np.where(a > 0, np.exp2(e - 8), 0.0)
    return np.maximum(TOL_O_BF16, half_ulp + 1e-3)


def gpu_forward(q, k, v, *, scale, causal, seqlens, out_dtype, variant=0, device="cuda"):
    """Copy CPU inputs to the GPU, run the HIP path, return CPU (O, LSE) and device outputs."""
    qd, kd, vd = (x.to(device).contiguous() for x in (q, k, v))
    sd = None if seqlens is None else seqlens.to(device=device, dtype=torch.int32).contiguous()
    o, lse = fa.forward(qd, kd, vd, scale=scale, causal=causal, seqlens=sd, out_dtype=out_dtype,
                        variant=variant)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def oracle_threads() -> int:
    """Host threads for oracle work: the CPUs this process may use, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def attention_ref_heads(q, k, v, scale, causal=False, seqlens=None, rows=None):
    """``oracle.attention_ref`` called once per (batch, head) on a thread pool, each call with a
    single-threaded BLAS; the results are stacked back to [B, H, R, d] and [B, H, R].  The
    oracle itself is unchanged: numpy releases the interpreter lock inside its array work, so the
    heads run side by side (full-size workloads would otherwise take minutes)."""
    B, H = q.shape[:2]
    r = None if rows is None else np.asarray(rows.cpu().numpy() if hasattr(rows, "numpy") else rows)

    def one(bh):
        b, h = divmod(bh, H)
        rr = None if r is None else (r if r.ndim == 1 else r[b:b + 1, h:h + 1])
        sl = None if seqlens is None else [int(seqlens[b])]
        return oracle.attention_ref(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], scale,
                                    causal=causal, seqlens=sl, rows=rr)

    with threadpoolctl.threadpool_limits(1), ThreadPoolExecutor(oracle_threads()) as ex:
        parts = list(ex.map(one, range(B * H)))
    O = np.stack([p[0][0, 0] for p in parts]).reshape(B, H, *parts[0][0].shape[2:])
    L = np.stack([p[1][0, 0] for p in parts]).reshape(B, H, -1)
    return O, L


def select_rows(x: torch.Tensor, rows) -> np.ndarray:
    """x [B, H, N, ...] -> rows per head [B, H, R, ...] (rows: None, [R] or [B, H, R])."""
    a = to_f64(x)
    if rows is None:
        return a
    r = np.asarray(rows)
    if r.ndim == 1:
        return a[:, :, r]
    B, H = a.shape[:2]
    return np.stack([np.stack([a[b, h, r[b, h]] for h in range(H)]) for b in range(B)])


def compare(o_gpu: torch.Tensor, lse_gpu: torch.Tensor, O_ref, LSE_ref, out_dtype, rows=None,
            label=""):
    """Assert the documented tolerances; return a dict of the measured errors."""
    o = select_rows(o_gpu, rows)
    lse = select_rows(lse_gpu, rows)
    assert o.shape == O_ref.shape, (o.shape, O_ref.shape)
    assert np.isfinite(o).all(), f"{label}: non-finite output"
    err = np.abs(o - O_ref)
    fin = np.isfinite(LSE_ref)
    assert np.array_equal(np.isfinite(lse), fin), f"{label}: LSE finiteness differs"
    assert np.all(lse[~fin] == LSE_ref[~fin]), f"{label}: -inf LSE differs"
    lse_err = np.abs(lse[fin] - LSE_ref[fin]) if fin.any() else np.zeros(1)
    res = {"max_abs_O": float(err.max()) if err.size else 0.0,
           "max_abs_LSE": float(lse_err.max()) if lse_err.size else 0.0}
    if out_dtype == torch.float32:
        assert res["max_abs_O"] <= TOL_O_F32, f"{label}: O err {res['max_abs_O']:.3e} > {TOL_O_F32}"
    else:
        bound = bf16_bound(O_ref)
        worst = float((err / bound).max()) if err.size else 0.0
        floor = np.abs(torch.from_numpy(O_ref).to(torch.bfloat16).double().numpy() - O_ref)
        res["bf16_floor"] = float(floor.max()) if floor.size else 0.0
        res["err_over_bound"] = worst
        assert worst <= 1.0, (f"{label}: O err {res['max_abs_O']:.3e} exceeds the per-element bound "
                              f"(ratio {worst:.3f}; rounding floor {res['bf16_floor']:.3e})")
    assert res["max_abs_LSE"] <= TOL_LSE, f"{label}: LSE err {res['max_abs_LSE']:.3e} > {TOL_LSE}"
    return res


def check_case(q, k, v, *, scale, causal=False, seqlens=None, out_dtype=torch.bfloat16, rows=None,
               variant=0, label=""):
    o, lse = gpu_forward(q, k, v, scale=scale, causal=causal, seqlens=seqlens, out_dtype=out_dtype,
                         variant=variant)
    sl = None if seqlens is None else seqlens.tolist()
    if q.shape[0] * q.shape[1] > 1 and q.shape[2] >= 1024:
        O_ref, LSE_ref = attention_ref_heads(q, k, v, scale, causal=causal, seqlens=sl, rows=rows)
    else:
        O_ref, LSE_ref = oracle.attention_ref(q, k, v, scale, causal=causal, seqlens=sl, rows=rows)
    return compare(o, lse, O_ref, LSE_ref, out_dtype, rows=rows, label=label)
