"""GPU parity of the packed variable-length forward (fa_fwd_varlen) against the fp64 oracle.

The HIP path is called through the C ABI (``forward_varlen``) on seeded packed inputs; the
expected values come from ``oracle.attention_varlen_ref`` alone (or, for long self-attention
sequences, from the square oracle on sampled rows, where the two alignments coincide).
Tolerances are those of the square forward: float32 output |dO| <= 2e-4, bf16 output within
max(1e-2, half a bf16 ulp + 1e-3) per element, LSE <= 1e-4.

Cases: ragged packed batches with empty sequences, more queries than keys and fewer, both
causal alignments and no mask; the tile kernel (more than 4 query rows) unsplit and with its
keys split into ranges merged afterwards (small grids); the decoding kernel (at most 4 query
rows) with one key range and with several merged ranges; the full-size decoding,
chunked-prefill and packed-mix workloads; isolation between neighbouring sequences; bitwise
determinism; and workspace reuse.
"""

import numpy as np
import pytest
import torch

import exact_tiled_attention_19_amd as fa
import oracle
from exact_tiled_attention_19_amd import workloads as W
from tests import parity_util as PU

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16
DEV = "cuda"
MASKS = {"none": (False, "bottom_right"), "causal_br": (True, "bottom_right"), "causal_tl": (True, "top_left")}


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    fa.load_library()


def run_gpu(q, k, v, cu_q, cu_k, lq, lk, scale, causal, align, out_dtype, workspace=None):
    o, lse = fa.forward_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cu_q.to(DEV), cu_k.to(DEV), max(lq), max(lk),
                               scale=scale, causal=causal, align=align, out_dtype=out_dtype, workspace=workspace)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def check(lq, lk, H, d, mask, out_dtype, seed, label):
    causal, align = MASKS[mask]
    q, k, v, cu_q, cu_k = W.random_packed(lq, lk, H, d, BF16, seed)
    scale = W.scale_for(d)
    print(f"[varlen] {label}", flush=True)
    o, lse = run_gpu(q, k, v, cu_q, cu_k, lq, lk, scale, causal, align, out_dtype)
    O_ref, L_ref = oracle.attention_varlen_ref(q, k, v, cu_q.tolist(), cu_k.tolist(), scale, causal=causal, align=align)
    res = PU.compare(o, lse, O_ref, L_ref, out_dtype, label=label)
    print(f"[varlen] {label}: {res}", flush=True)
    return o, lse


# tile-kernel shapes (longest query sequence > 4 rows): empty sequences, Lq > Lk, Lq < Lk,
# lengths across several 128-row tiles and 64-key tiles with ragged tails
PREFILL = {
    "mixed": ([130, 0, 7, 300], [130, 64, 9, 200]),
    "self": ([1, 129, 256, 77], [1, 129, 256, 77]),
    "chunk": ([64, 5], [1000, 0]),
    "overfull": ([200, 33], [70, 1]),
}


@pytest.mark.parametrize("out_dtype", [BF16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask", list(MASKS))
@pytest.mark.parametrize("shape", list(PREFILL))
def test_prefill_kernel(shape, mask, d, out_dtype):
    lq, lk = PREFILL[shape]
    check(lq, lk, 2, d, mask, out_dtype, seed=100 + d, label=f"prefill {shape} d={d} {mask} {out_dtype}")


# decoding-kernel shapes (longest query sequence <= 4 rows): one key range (<= 512 keys) and
# several ranges merged; empty key sets; more query rows than keys
DECODE = {
    "one_row_split": ([1] * 5, [0, 1, 300, 4097, 64]),
    "one_row_single_range": ([1, 1, 1], [200, 17, 0]),
    "four_rows_split": ([1, 4, 3, 2], [5000, 3, 256, 1]),
    "four_rows_single_range": ([4, 2], [40, 7]),
}


@pytest.mark.parametrize("out_dtype", [BF16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask", list(MASKS))
@pytest.mark.parametrize("shape", list(DECODE))
def test_decode_kernel(shape, mask, d, out_dtype):
    lq, lk = DECODE[shape]
    check(lq, lk, 3, d, mask, out_dtype, seed=200 + d, label=f"decode {shape} d={d} {mask} {out_dtype}")


# tile-kernel shapes whose grid is small enough (at most 128 tiles, at least 1024 keys) that
# the keys are split into ranges: ranges past a sequence's keys (empty), ranges above the causal
# diagonal, an empty query sequence, key counts off the 64-key tile, more queries than keys
SPLIT = {
    "chunk": ([300, 77], [3000, 1100]),
    "self": ([1500, 129], [1500, 129]),
    "ragged": ([1, 257, 0], [2049, 4000, 700]),
    "more_q": ([2000], [1030]),
}


@pytest.mark.parametrize("out_dtype", [BF16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask", list(MASKS))
@pytest.mark.parametrize("shape", list(SPLIT))
def test_prefill_kernel_split_keys(shape, mask, d, out_dtype):
    lq, lk = SPLIT[shape]
    H = 2
    n = fa.varlen_workspace_size(len(lq), H, max(lq), max(lk), d)
    assert n > 0, "the shape should take the split path"
    check(lq, lk, H, d, mask, out_dtype, seed=60 + d, label=f"split {shape} mask={mask} d={d} out={out_dtype} ({n} B)")


def test_prefill_kernel_paired_launch():
    """Enough causal tiles (32 sequences x 64 heads x 3 tiles) that the launch pairs tiles
    (n-1-t, t) of each sequence; ragged lengths from 1 to 300, every row checked."""
    lq = list(W.draw_lengths(33, 32, 1, 300))
    lq[0] = 300
    check(lq, lq, 64, 64, "causal_br", BF16, seed=34, label="prefill paired launch")


@pytest.mark.parametrize("name", ["decode_c2kv", "decode_c4kv"])
def test_decode_workloads_full_size(name):
    w = W.PACKED[name]
    check(list(w.lq), list(w.lk), w.H, w.d, "causal_br" if w.causal else "none", BF16, w.seed, f"workload {name}")


@pytest.mark.parametrize("name", ["chunked_prefill", "varlen_mix", "single_4k_d64", "single_8k_d128"])
def test_packed_workloads_full_size_sampled(name):
    """Full-size packed prefill: every sequence runs on the GPU; the first `sample_seqs`
    sequences are checked (chunked prefill: all their rows through the variable-length oracle;
    packed self-attention: 512 sampled rows per head through the square oracle, where both
    alignments coincide)."""
    w = W.PACKED[name]
    q, k, v, cu_q, cu_k = W.random_packed(w.lq, w.lk, w.H, w.d, BF16, w.seed)
    print(f"[varlen] workload {name}", flush=True)
    o, lse = run_gpu(q, k, v, cu_q, cu_k, w.lq, w.lk, w.scale, w.causal, w.align, BF16)
    g = torch.Generator("cpu").manual_seed(w.seed + 1000)
    for b in range(w.sample_seqs):
        qs, qe, ks, ke = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        if w.lq[b] != w.lk[b]:
            O_ref, L_ref = oracle.attention_varlen_ref(q[qs:qe], k[ks:ke], v[ks:ke], [0, qe - qs], [0, ke - ks],
                                                       w.scale, causal=w.causal, align=w.align)
            res = PU.compare(o[qs:qe], lse[:, qs:qe], O_ref, L_ref, BF16, label=f"{name} seq {b}")
        else:
            L = qe - qs
            rows = torch.sort(torch.randperm(L, generator=g)[:512]).values.numpy()
            qb, kb, vb = (x.permute(1, 0, 2).unsqueeze(0).contiguous() for x in (q[qs:qe], k[ks:ke], v[ks:ke]))
            O_ref, L_ref = oracle.attention_ref(qb, kb, vb, w.scale, causal=w.causal, rows=rows)
            og = o[qs:qe].permute(1, 0, 2)[:, rows].unsqueeze(0)
            lg = lse[:, qs:qe][:, rows].unsqueeze(0)
            res = PU.compare(og, lg, O_ref, L_ref, BF16, label=f"{name} seq {b}")
        print(f"[varlen] {name} seq {b}: {res}", flush=True)


@pytest.mark.parametrize("max_q_rows", [300, 1])
def test_sequences_are_isolated(max_q_rows):
    """Extreme finite values in a neighbouring sequence's keys and values change nothing."""
    lq = [max_q_rows, max_q_rows, max_q_rows]
    lk = [150, 90, 150]
    q, k, v, cu_q, cu_k = W.random_packed(lq, lk, 2, 128, BF16, seed=31)
    scale = W.scale_for(128)
    a = run_gpu(q, k, v, cu_q, cu_k, lq, lk, scale, True, "bottom_right", torch.float32)
    k2, v2 = k.clone(), v.clone()
    k2[150:240] = 3.0e38
    v2[150:240] = -3.0e38
    b = run_gpu(q, k2, v2, cu_q, cu_k, lq, lk, scale, True, "bottom_right", torch.float32)
    for s in (slice(0, max_q_rows), slice(2 * max_q_rows, 3 * max_q_rows)):
        assert torch.equal(a[0][s], b[0][s])
        assert torch.equal(a[1][:, s], b[1][:, s])


@pytest.mark.parametrize("lq,lk", [([300, 41], [500, 800]), ([1, 1, 1, 1], [6000, 5, 9000, 300]),
                                   ([300, 41], [3000, 1100])])
def test_bitwise_determinism_and_workspace_reuse(lq, lk):
    q, k, v, cu_q, cu_k = W.random_packed(lq, lk, 4, 64, BF16, seed=32)
    scale = W.scale_for(64)
    n = fa.varlen_workspace_size(len(lq), 4, max(lq), max(lk), 64)
    ws = torch.full((max(n, 16) + 4096,), 255, dtype=torch.uint8, device=DEV)   # stale contents
    a = run_gpu(q, k, v, cu_q, cu_k, lq, lk, scale, True, "bottom_right", BF16, workspace=ws)
    b = run_gpu(q, k, v, cu_q, cu_k, lq, lk, scale, True, "bottom_right", BF16, workspace=ws)
    c = run_gpu(q, k, v, cu_q, cu_k, lq, lk, scale, True, "bottom_right", BF16)
    assert torch.equal(a[0], b[0]) and torch.equal(a[0], c[0])
    assert torch.equal(a[1], b[1]) and torch.equal(a[1], c[1])


def test_errors_surface():
    x = torch.zeros(16, 2, 64, dtype=BF16, device=DEV)
    cu = torch.tensor([0, 16], dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        fa.forward_varlen(x, x, x, cu, cu, 16, 16, align="diagonal")
    with pytest.raises(fa.FaInvalidArgument):
        fa.forward_varlen(x, x, x, cu, cu, 16, 16, out=x)          # o aliases q
    ws = torch.empty(8, dtype=torch.uint8, device=DEV)
    y = torch.zeros(8192, 2, 64, dtype=BF16, device=DEV)
    cuk = torch.tensor([0, 8192], dtype=torch.int32, device=DEV)
    qd = torch.zeros(1, 2, 64, dtype=BF16, device=DEV)
    cuq = torch.tensor([0, 1], dtype=torch.int32, device=DEV)
    with pytest.raises(fa.FaInvalidArgument):
        fa.forward_varlen(qd, y, y, cuq, cuk, 1, 8192, workspace=ws)   # workspace too small
