#!/usr/bin/env python3
"""Benchmark of the fused exact-attention forward on one MI355X.

One step = one fused forward (one kernel launch) over the whole workload, inputs already
resident in device memory.  Prints one JSON line:

  value      whole-job throughput in TFLOP/s, counting 4*B*H*N^2*d FLOP per forward
             (halved under the causal mask);
  roofline   the kernel's achieved TFLOP/s per launch (same FLOP count / the average launch
             duration, timed with HIP events on the launch stream) against the MI355X dense
             bf16 MFMA peak, plus HBM traffic per launch from rocprofv3 FETCH_SIZE/WRITE_SIZE
             counters when the recorded counters match the current kernel sources;
  cpu_baseline  the fp64 CPU oracle timed on this host on a bounded sample of the same
             workload (seed-chosen query rows of every head), scaled to TFLOP/s.

Packed variable-length workloads (--workload decode_c2kv | decode_c4kv | chunked_prefill |
varlen_mix | single_4k_d64 | single_8k_d128) time fa_fwd_varlen instead: decoding steps are
bound by the K/V stream and are reported in GB/s against the HBM peak; packed prefill in
TFLOP/s counting 4*d FLOP per visible (query, key) pair.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2] [--no-cpu-baseline]
       python bench.py --calibrate-copy      (a plain conversion copy of known size, for scaling
                                              the FETCH_SIZE / WRITE_SIZE counters to bytes)
"""

from __future__ import annotations

import argparse
import dataclasses
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s and % of bf16 MFMA peak, N=4k–128k, d=64/128, 1 GPU"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_F32_TFLOPS = 157.3     # MI355X dense fp32 MFMA
PEAK_FP8_TFLOPS = 5033.2    # MI355X dense fp8 MFMA: 256 CU x 8192 FLOP/clk x 2.4 GHz
# 8-bit inputs: S = Q K^T (half the counted FLOP) runs on fp8 MFMA, O += P V (the other half) on
# bf16 MFMA, so the time at peak is F/2 / fp8 peak + F/2 / bf16 peak
PEAK_FP8_BF16_MIXED_TFLOPS = round(1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS), 1)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILES = os.path.join(ROOT, "profiles", "*_traffic.txt")
# the sources the forward kernels are compiled from (the backward's own header is not among them:
# recorded forward counters stay valid across backward-only changes)
KERNEL_SOURCES = ["fa_api.hip", "fa_fp8.hip", "fa_fwd_bf16.h", "fa_fwd_ksplit.h", "fa_fwd_bf16_pipe.h", "fa_fwd_f32.h", "fa_sched.h",
                  "fa_decode_bf16.h", "fa_dropout.h"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for s in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "exact_tiled_attention_19_amd", "csrc", s), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def compulsory_bytes(B, H, N, d, in_bytes, out_bytes) -> int:
    """Q, K, V read once, O and the float32 LSE written once (the N x N scores never are)."""
    return B * H * (3 * N * d * in_bytes + N * d * out_bytes + 4 * N)


def counted_flops(B, H, N, d, causal) -> float:
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def recorded_traffic(workload: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary for this workload, or
    None when there is none or it predates the current kernel sources."""
    for path in sorted(glob.glob(TRAFFIC_FILES)):
        vals = {}
        with open(path) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    key, val = line.split(":", 1)
                    vals[key.strip()] = val.strip()
        if vals.get("workload") != workload or vals.get("kernel_source_sha256_16") != kernel_source_hash():
            continue
        try:
            return float(vals["hbm_bytes_per_launch"])
        except (KeyError, ValueError):
            continue
    return None


def visible_pairs(lq, lk, causal: bool, align: str) -> int:
    """(query, key) pairs the mask lets through, summed over the packed sequences."""
    total = 0
    for a, b in zip(lq, lk):
        if not causal:
            total += a * b
            continue
        dlt = b - a if align == "bottom_right" else 0
        for i in range(a):   # row i sees keys 0 .. min(b - 1, i + dlt)
            total += max(0, min(b, i + dlt + 1))
    return total


def time_steps(step, steps: int, warmup: int, dev):
    """W untimed steps, then K timed ones; returns (wall seconds, mean per-step HIP-event seconds)."""
    import torch
    print(f"[bench] warmup {warmup}", file=sys.stderr, flush=True)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    print(f"[bench] timing {steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [e0.elapsed_time(e1) for e0, e1 in evs]
    return wall, sum(launch_ms) / len(launch_ms) / 1e3


def bench_packed(args, w) -> int:
    """fa_fwd_varlen on a packed workload: decoding shapes against the HBM peak (bytes of Q, K,
    V read and O, LSE written once), packed prefill against the bf16 MFMA peak."""
    import torch
    import exact_tiled_attention_19_amd as fa
    from exact_tiled_attention_19_amd import workloads as W
    dev = torch.device("cuda", 0)
    print(f"[bench] generating {w.name} inputs", file=sys.stderr, flush=True)
    qh, kh, vh, cqh, ckh = W.random_packed(w.lq, w.lk, w.H, w.d, torch.bfloat16, w.seed)
    q, k, v, cu_q, cu_k = (t.to(dev) for t in (qh, kh, vh, cqh, ckh))
    mq, mk = max(w.lq), max(w.lk)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.H, q.shape[0]), dtype=torch.float32, device=dev)
    nws = fa.varlen_workspace_size(len(w.lq), w.H, mq, mk, w.d)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev) if nws else None
    torch.cuda.synchronize()

    def step():
        fa.forward_varlen(q, k, v, cu_q, cu_k, mq, mk, scale=w.scale, causal=w.causal, align=w.align,
                          out=o, lse_out=lse, workspace=ws)

    wall, avg_launch_s = time_steps(step, args.steps, args.warmup, dev)
    decode = mq <= 4
    Tq, Tk = sum(w.lq), sum(w.lk)
    nbytes = w.H * w.d * 2 * (Tq + 2 * Tk) + w.H * w.d * 2 * Tq + 4 * w.H * Tq
    flops = 4.0 * w.d * w.H * visible_pairs(w.lq, w.lk, w.causal, w.align)
    mask_name = f"causal {w.align.replace('_', '-')}" if w.causal else "none"
    workload_id = f"{w.name}:{'causal-' + w.align if w.causal else 'none'}:bf16-out"
    if decode:
        metric, unit, bound, peak = ("attention decode GB/s (Q, K, V read and O, LSE written once), 1 GPU",
                                     "GB/s", "hbm", PEAK_HBM_GBS)
        value = nbytes / (wall / args.steps) / 1e9
        achieved = nbytes / avg_launch_s / 1e9
    else:
        metric, unit, bound, peak = ("attention fwd TFLOP/s, packed variable-length sequences (4*d FLOP per "
                                     "visible query-key pair), 1 GPU", "TFLOP/s", "mfma", PEAK_BF16_TFLOPS)
        value = flops / (wall / args.steps) / 1e12
        achieved = flops / avg_launch_s / 1e12
    res = {
        "metric": metric, "value": round(value, 3), "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded normal Q, K, V of the workload's packed shape; no dataset)",
        "config": {
            "workload": f"{w.name}: {w.description}; {mask_name} mask; bf16 in, bf16 out, fp32 LSE",
            "sequences": len(w.lq), "H": w.H, "d": w.d, "tokens_q": Tq, "tokens_k": Tk,
            "max_seqlen_q": mq, "max_seqlen_k": mk, "kernel": ("decode (split keys + merge)" if decode else
                                                  "tile, keys split into ranges + merge" if nws else "tile"),
            "workspace_bytes": nws, "flop_per_step": flops, "compulsory_bytes_per_step": nbytes,
        },
        "roofline": {
            "bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 5), "traffic": recorded_traffic(workload_id),
            "kernel_avg_ms": round(avg_launch_s * 1e3, 5),
        },
    }
    if nws:
        res["roofline"]["note"] = "HIP events bracket both kernels of a step (the key ranges and their merge)"
    if not args.no_cpu_baseline:
        import oracle
        try:
            from threadpoolctl import threadpool_info
            threads = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"),
                          default=1)
        except Exception:  # pragma: no cover
            threads = os.cpu_count() or 1
        # bounded sample: whole decoding steps, or the first sequences of a packed prefill batch
        nseq = len(w.lq) if decode else max(1, min(len(w.lq), 2))
        sq, sk = list(w.lq[:nseq]), list(w.lk[:nseq])
        qs, ks = sum(sq), sum(sk)
        print(f"[bench] timing the fp64 oracle on {nseq} sequence(s)", file=sys.stderr, flush=True)
        t0 = time.perf_counter()
        oracle.attention_varlen_ref(qh[:qs], kh[:ks], vh[:ks], [0] + list(torch.cumsum(torch.tensor(sq), 0).tolist()),
                                    [0] + list(torch.cumsum(torch.tensor(sk), 0).tolist()), w.scale,
                                    causal=w.causal, align=w.align)
        dt = time.perf_counter() - t0
        if decode:
            sb = w.H * w.d * 2 * (qs + 2 * ks) + w.H * w.d * 2 * qs + 4 * w.H * qs
            cv = sb / dt / 1e9
        else:
            cv = 4.0 * w.d * w.H * visible_pairs(sq, sk, w.causal, w.align) / dt / 1e12
        res["cpu_baseline"] = {"value": round(cv, 6), "unit": unit, "cores": int(threads), "kind": "oracle",
                               "sample": f"{nseq} of the {len(w.lq)} sequences, all heads, fp64 numpy, "
                                         f"{dt:.1f} s wall"}
    print(json.dumps(res), flush=True)
    return 0


def cpu_baseline(w, x, rows_per_head: int, descales=None):
    """Time the fp64 oracle on `rows_per_head` seed-chosen query rows of every head (8-bit
    inputs: the 8-bit oracle with the given descales)."""
    import numpy as np  # noqa: F401
    import torch
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"),
                      default=1)
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    g = torch.Generator("cpu").manual_seed(12345)
    rows = torch.stack([torch.stack([torch.sort(torch.randperm(w.N, generator=g)[:rows_per_head]).values
                                     for _ in range(w.H)]) for _ in range(w.B)])
    causal = bool(w.mask_kinds[0] & 1)
    seq = x.seqlens.tolist() if x.seqlens is not None else None
    t0 = time.perf_counter()
    if descales is None:
        oracle.attention_ref(x.q, x.k, x.v, x.scale, causal=causal, seqlens=seq, rows=rows)
    else:
        oracle.attention_fp8_ref(x.q, x.k, x.v, *descales, x.scale, causal=causal, seqlens=seq, rows=rows)
    dt = time.perf_counter() - t0
    # counted FLOP of the sampled rows: each row carries 4*d*(keys it is charged for); the
    # causal convention charges a row N/2 keys on average, so a uniform sample of R rows per
    # head carries R/N of the whole workload's counted FLOP.
    frac = rows_per_head / w.N
    flops = counted_flops(w.B, w.H, w.N, w.d, causal) * frac
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{rows_per_head} seed-chosen query rows of each of the {w.B * w.H} heads "
                      f"({frac:.4%} of the workload's counted FLOP), fp64 numpy, {dt:.1f} s wall"}


COPY_ELEMS = 1 << 28   # 256 Mi elements: 1 GiB of fp32 read, 512 MiB of bf16 written


def calibrate_copy(steps: int) -> int:
    """Run a plain elementwise fp32 -> bf16 copy whose HBM traffic is known exactly
    (4 bytes read and 2 bytes written per element, 1.5 GiB per launch, far above the L2 and the
    256 MiB last-level cache), so a profiler's byte counters can be scaled to true bytes."""
    import torch
    dev = torch.device("cuda", 0)
    src = torch.ones(COPY_ELEMS, dtype=torch.float32, device=dev)
    dst = torch.empty(COPY_ELEMS, dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "fp32->bf16 copy", "elements": COPY_ELEMS,
                      "read_bytes": 4 * COPY_ELEMS, "write_bytes": 2 * COPY_ELEMS,
                      "launches": steps}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed launches first: the shader clock settles over the first ~100 ms")
    ap.add_argument("--workload", default="c2",
                    help="c0..c4 (default c2, the roofline workload), a short-sequence HBM probe "
                         "bw<N>d<d> with N in 128/256/512 and d in 64/128, or a packed workload "
                         "(decode_c2kv, decode_c4kv, chunked_prefill, varlen_mix, single_4k_d64, "
                         "single_8k_d128)")
    ap.add_argument("--mask", type=int, default=None, help="override the workload's mask bits")
    ap.add_argument("--out-dtype", default=None, choices=[None, "bf16", "f32"])
    ap.add_argument("--variant", type=int, default=0)
    ap.add_argument("--qk-gain", type=float, default=None,
                    help="override the workload's Q/K gain (c3 uses 3: logit std ~ 9; 1 gives flat rows)")
    ap.add_argument("--cpu-rows", type=int, default=6144, help="oracle rows per head for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--dropout", type=float, default=None,
                    help="time the forward with dropout of this probability on the attention weights "
                         "(fa_fwd_dropout, Philox seed 1234)")
    ap.add_argument("--fp8", action="store_true",
                    help="FP8 E4M3 inputs (fa_fwd_fp8): the workload's normals quantised per tensor "
                         "with amax descales")
    ap.add_argument("--bwd", action="store_true",
                    help="time the backward pass (fa_bwd: dQ, dK, dV) instead of the forward")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only the known-size copy used to calibrate the byte counters")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this benchmark measures one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); the forward pass shards over (batch, head) with no "
              f"communication, so multi-GPU throughput is N x the one-GPU value by construction "
              f"and is not measured here.", file=sys.stderr)
        return 2

    import torch
    import exact_tiled_attention_19_amd as fa
    from exact_tiled_attention_19_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    if args.calibrate_copy:
        return calibrate_copy(args.steps)
    fa.load_library()
    if args.workload in W.PACKED:
        return bench_packed(args, W.PACKED[args.workload])
    probe = args.workload in W.PROBES
    w = W.PROBES[args.workload] if probe else W.WORKLOADS[args.workload]
    mask = w.mask_kinds[0] if args.mask is None else args.mask
    causal = bool(mask & W.MASK_CAUSAL)
    out_dtype = w.out_dtypes[0] if args.out_dtype is None else (
        torch.bfloat16 if args.out_dtype == "bf16" else torch.float32)
    print(f"[bench] generating {w.name} inputs", file=sys.stderr, flush=True)
    if args.qk_gain is not None:
        w = dataclasses.replace(w, qk_gain=args.qk_gain)
    x = W.make_inputs(w, mask_kind=mask)
    dev = torch.device("cuda", 0)
    if args.fp8 and (args.bwd or args.dropout is not None or probe or w.in_dtype != torch.bfloat16):
        print("bench.py: --fp8 times the forward of a bf16 workload (c1..c4), without --bwd or --dropout",
              file=sys.stderr)
        return 1
    if args.fp8:
        q8, k8, v8, descales = W.random_qkv_fp8(w.B, w.H, w.N, w.d, w.seed, w.qk_gain)
        x = dataclasses.replace(x, q=q8, k=k8, v=v8)
    q, k, v = (t.to(dev) for t in (x.q, x.k, x.v))
    seq = x.seqlens.to(dev) if (mask & W.MASK_KEY_PADDING) else None
    o = torch.empty(q.shape, dtype=out_dtype, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step():
        fa.forward(q, k, v, scale=x.scale, causal=causal, seqlens=seq, out_dtype=out_dtype,
                   out=o, lse_out=lse, variant=args.variant)

    if args.fp8:
        def step():
            fa.forward_fp8(q, k, v, descale_q=descales[0], descale_k=descales[1], descale_v=descales[2],
                           scale=x.scale, causal=causal, seqlens=seq, out_dtype=out_dtype, out=o, lse_out=lse)

    if args.dropout is not None:
        def step():
            fa.forward_dropout(q, k, v, args.dropout, 1234, 0, scale=x.scale, causal=causal, seqlens=seq,
                               out_dtype=out_dtype, out=o, lse_out=lse)

    if args.bwd:
        # the forward's bf16 output and LSE, and a seeded upstream gradient of the same shape
        if q.dtype != torch.bfloat16:
            print("bench.py: the backward pass takes bf16 inputs", file=sys.stderr)
            return 1
        o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
        out_dtype = torch.bfloat16
        step()
        g = torch.Generator("cpu").manual_seed(w.seed + 1000)
        dout = torch.randn(q.shape, generator=g).to(torch.bfloat16).to(dev)
        grads = tuple(torch.empty(q.shape, dtype=torch.float32, device=dev) for _ in range(3))
        delta = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)

        drop = None if args.dropout is None else (args.dropout, 1234, 0)   # the forward's mask

        def step():
            fa.backward(q, k, v, o, lse, dout, scale=x.scale, causal=causal, seqlens=seq, out=grads,
                        delta=delta, dropout=drop)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [e0.elapsed_time(e1) for e0, e1 in evs]
    avg_launch_s = sum(launch_ms) / len(launch_ms) / 1e3
    ms_per_step = wall / args.steps * 1e3

    flops = counted_flops(w.B, w.H, w.N, w.d, causal)
    if args.bwd:   # five products of the forward's size (S, dP, dV, dK, dQ): 2.5x the forward
        flops *= 2.5
    value = flops / (wall / args.steps) / 1e12
    fp32 = w.in_dtype == torch.float32
    nbytes = compulsory_bytes(w.B, w.H, w.N, w.d, 4 if fp32 else 1 if args.fp8 else 2,
                              4 if out_dtype == torch.float32 else 2)
    if probe:   # HBM-bound: compulsory bytes per launch against the HBM peak
        bound, unit, peak, achieved = "hbm", "GB/s", PEAK_HBM_GBS, nbytes / avg_launch_s / 1e9
    else:       # MFMA-bound: counted FLOP per launch against the dense MFMA peak of the input dtype
        bound, unit = "mfma", "TFLOP/s"
        peak = PEAK_F32_TFLOPS if fp32 else PEAK_FP8_BF16_MIXED_TFLOPS if args.fp8 else PEAK_BF16_TFLOPS
        achieved = flops / avg_launch_s / 1e12
    mask_name = {0: "none", 1: "causal", 2: "key_padding", 3: "causal+key_padding"}[mask]
    workload_id = (f"{w.name}:{mask_name}:{'fp8-in:' if args.fp8 else ''}"
                   f"{'f32' if out_dtype == torch.float32 else 'bf16'}-out")
    traffic = recorded_traffic(workload_id)

    res = {
        "metric": (METRIC if not args.bwd else "attention bwd TFLOP/s (dQ, dK, dV; 2.5x the forward's FLOP), 1 GPU")
        + (f", dropout p={args.dropout}" if args.dropout is not None else ""),
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if fp32 else "fp8-e4m3 (Q K^T), bf16 (P V)" if args.fp8 else "bf16",
        "data": "synthetic (seeded normal Q, K, V of the workload's shape; no dataset)",
        "config": {
            "workload": (f"{w.name}: B={w.B} H={w.H} N={w.N} d={w.d} {mask_name} mask, "
                         + (f"Q/K gain {w.qk_gain:g}, " if w.qk_gain != 1.0 else "")
                         + f"{'fp32' if fp32 else 'fp8 e4m3 (per-tensor descales)' if args.fp8 else 'bf16'} in, "
                         + f"{'fp32' if out_dtype == torch.float32 else 'bf16'} out, fp32 LSE"),
            "B": w.B, "H": w.H, "N": w.N, "d": w.d, "mask": mask_name,
            "flop_per_step": flops, "compulsory_bytes_per_step": nbytes, "variant": args.variant,
            "pass": "backward" if args.bwd else "forward",
            "dropout": args.dropout,
        },
        "roofline": {
            "bound": bound,
            "achieved": round(achieved, 3),
            "peak": peak,
            "unit": unit,
            "frac": round(achieved / peak, 5),
            "traffic": traffic,
            "kernel_avg_ms": round(avg_launch_s * 1e3, 5),
        },
    }
    if args.bwd:
        res["roofline"]["note"] = ("three kernels per step (row term, dK/dV, dQ); achieved counts the pass's "
                                   "2.5x-forward FLOP over their combined time, which executes 3.5x")
        res["roofline"]["traffic"] = None
    if not args.no_cpu_baseline and not args.bwd and args.dropout is None:
        print(f"[bench] timing the fp64 oracle on {args.cpu_rows} rows per head", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w, x, min(args.cpu_rows, w.N), descales if args.fp8 else None)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
