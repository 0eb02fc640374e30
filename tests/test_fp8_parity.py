"""GPU parity of the FP8 E4M3 forward (fa_fwd_fp8) against the fp64 oracle on the decoded inputs.

Bounds.  V is widened to bf16 without rounding and the value product is the bf16 path's, so the
bf16 path's bounds (tests/parity_util.py) are the base: float32 output O <= 2e-4; bf16 output
per element max(1e-2, half a bf16 ulp + 1e-3); LSE <= 1e-4.  On top of them comes the score
error of the 8-bit matrix instruction (v_mfma_f32_32x32x64_f8f6f4).  Its 64 products are exact,
but they are summed in groups whose partial sums keep only about 14 significant bits
(truncated); the add into the float32 accumulator is exact.  Measured on MI355X with one
instruction and exact host sums: 2^16 + 63 x 1 gives 2^16 + 56, 2^16 + 63 x 0.5 gives 2^16 + 28,
2^20 (accumulator) + 64 x 1 is exact; random operands err by at most 2^-13.2 of sum_k |a_k b_k|.
So score s_ij carries at most delta_ij = ACC_REL * scale * sum_k |q_ik k_jk| with ACC_REL =
2^-11 (four times the worst measured), and with D_i = max over visible j of delta_ij:
  |LSE_i error| <= 1e-4 + D_i   (the log-sum-exp moves by at most the largest score change);
  |O_id error|  <= base + (exp(2 D_i) - 1) * max over visible j of |v_jd|
(each weight changes by at most the factor exp(+-2 D_i)).  For unit-variance logits D_i is a
few 1e-5 and the base bounds decide.

* Seeded sweeps over several 128-row query tiles and 64-key tiles with ragged tails, both head
  widths, every mask, both output types, with per-tensor amax descales.
* Descale properties through the kernel: doubling the Q descale equals doubling the scale; the
  V descale scales O and leaves LSE alone; an all-zero Q gives the mean of the visible V rows.
* The c2 shape (B=4, H=16, N=8192, d=128, causal) at full size in the eight-wave launch the
  benchmark times, checked on seed-chosen rows.
"""

import numpy as np
import pytest
import torch

import exact_tiled_attention_19_amd as fa
import oracle
from exact_tiled_attention_19_amd import workloads as W
from tests.parity_util import TOL_LSE, TOL_O_F32, bf16_bound, select_rows, to_f64

pytestmark = pytest.mark.gpu

BF16, F32 = torch.bfloat16, torch.float32
MASKS = {"none": (False, False), "causal": (True, False), "pad": (False, True), "causal_pad": (True, True)}


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    fa.load_library()


def _run(q8, k8, v8, ds, *, scale, causal=False, seqlens=None, out_dtype=BF16):
    dev = "cuda"
    sd = None if seqlens is None else seqlens.to(device=dev, dtype=torch.int32)
    o, lse = fa.forward_fp8(q8.to(dev), k8.to(dev), v8.to(dev), descale_q=ds[0], descale_k=ds[1], descale_v=ds[2],
                            scale=scale, causal=causal, seqlens=sd, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


ACC_REL = 2.0 ** -11


def _row_bounds(q8, k8, v8, ds, scale, causal, seqlens, rows):
    """Per query row: D_i (largest score error bound over visible keys) and, per dimension, the
    largest |v_jd| over visible keys.  Shapes [B, H, R] and [B, H, R, d]."""
    q = np.abs(oracle.dequantize(q8, ds[0]))
    k = np.abs(oracle.dequantize(k8, ds[1]))
    v = np.abs(oracle.dequantize(v8, ds[2]))
    B, H, N, d = q.shape
    r_all = np.arange(N) if rows is None else None
    D = []
    VM = []
    for b in range(B):
        L = N if seqlens is None else int(min(max(int(seqlens[b]), 0), N))
        Db, Vb = [], []
        for h in range(H):
            r = r_all if rows is None else np.asarray(rows)[b, h] if np.asarray(rows).ndim == 3 else np.asarray(rows)
            vis = oracle.visible_keys(r, L, causal, N)
            a = ACC_REL * abs(scale) * (q[b, h, r] @ k[b, h].T)                  # [R, N]
            Db.append(np.where(vis, a, 0.0).max(axis=1) if N else np.zeros(len(r)))
            # the visible keys of a row are a prefix 0 .. n_i - 1 of the keys
            n_vis = vis.sum(axis=1)
            pref = np.maximum.accumulate(v[b, h], axis=0) if N else np.zeros((0, d))
            Vb.append(np.where((n_vis > 0)[:, None], pref[np.maximum(n_vis - 1, 0)] if N else 0.0, 0.0))
        D.append(Db)
        VM.append(Vb)
    return np.array(D), np.array(VM)


def _check(q8, k8, v8, ds, *, scale, causal=False, seqlens=None, out_dtype=BF16, rows=None, label=""):
    o, lse = _run(q8, k8, v8, ds, scale=scale, causal=causal, seqlens=seqlens, out_dtype=out_dtype)
    sl = None if seqlens is None else seqlens.tolist()
    O_ref, L_ref = oracle.attention_fp8_ref(q8, k8, v8, *ds, scale, causal=causal, seqlens=sl, rows=rows)
    D, VM = _row_bounds(q8, k8, v8, ds, scale, causal, sl, rows)
    o64, l64 = select_rows(o, rows), select_rows(lse, rows)
    assert np.isfinite(o64).all(), f"{label}: non-finite output"
    fin = np.isfinite(L_ref)
    assert np.array_equal(np.isfinite(l64), fin) and np.all(l64[~fin] == L_ref[~fin]), f"{label}: -inf LSE differs"
    base = np.full(O_ref.shape, TOL_O_F32) if out_dtype == F32 else bf16_bound(O_ref)
    o_bound = base + np.expm1(2 * D)[..., None] * VM
    l_bound = TOL_LSE + D
    o_ratio = float((np.abs(o64 - O_ref) / o_bound).max()) if O_ref.size else 0.0
    l_ratio = float((np.abs(l64[fin] - L_ref[fin]) / l_bound[fin]).max()) if fin.any() else 0.0
    res = {"max_abs_O": float(np.abs(o64 - O_ref).max()) if O_ref.size else 0.0,
           "max_abs_LSE": float(np.abs(l64[fin] - L_ref[fin]).max()) if fin.any() else 0.0,
           "max_score_bound": float(D.max()) if D.size else 0.0, "O_err_over_bound": o_ratio,
           "LSE_err_over_bound": l_ratio}
    print(f"[fp8] {label}: " + ", ".join(f"{k}={v:.3e}" for k, v in res.items()), flush=True)
    assert o_ratio <= 1.0, f"{label}: O error exceeds its bound (ratio {o_ratio:.3f})"
    assert l_ratio <= 1.0, f"{label}: LSE error exceeds its bound (ratio {l_ratio:.3f})"
    return res


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 17, 64, 65, 129, 300, 1000])
@pytest.mark.parametrize("mask", list(MASKS))
def test_sweep_fp8(N, d, mask):
    causal, pad = MASKS[mask]
    B, H = 2, 2
    q8, k8, v8, ds = W.random_qkv_fp8(B, H, N, d, seed=3000 + N + d)
    seq = None
    if pad:
        g = torch.Generator("cpu").manual_seed(N + 11)
        seq = torch.randint(0, N + 1, (B,), generator=g, dtype=torch.int32)
    for out_dtype in (BF16, F32):
        label = f"N={N} d={d} mask={mask} out={out_dtype}"
        print(f"[case] {label}", flush=True)
        _check(q8, k8, v8, ds, scale=W.scale_for(d), causal=causal, seqlens=seq, out_dtype=out_dtype, label=label)


@pytest.mark.parametrize("d", [64, 128])
def test_large_logits_fp8(d):
    """Logit std about 9 (Q, K normals times 3 before quantising): peaked rows."""
    q8, k8, v8, ds = W.random_qkv_fp8(1, 2, 517, d, seed=31, qk_gain=3.0)
    for out_dtype in (BF16, F32):
        _check(q8, k8, v8, ds, scale=W.scale_for(64), out_dtype=out_dtype, label=f"peaked d={d} out={out_dtype}")


def test_descale_properties_fp8():
    q8, k8, v8, ds = W.random_qkv_fp8(1, 2, 333, 128, seed=41)
    s = W.scale_for(128)
    o1, l1 = _run(q8, k8, v8, (2 * ds[0], ds[1], ds[2]), scale=s, causal=True, out_dtype=F32)
    o2, l2 = _run(q8, k8, v8, ds, scale=2 * s, causal=True, out_dtype=F32)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)     # the same float32 multiplier reaches the kernel
    o3, l3 = _run(q8, k8, v8, (ds[0], ds[1], 0.25 * ds[2]), scale=s, causal=True, out_dtype=F32)
    o4, l4 = _run(q8, k8, v8, ds, scale=s, causal=True, out_dtype=F32)
    assert torch.equal(l3, l4)
    assert torch.allclose(o3, 0.25 * o4, rtol=1e-6, atol=0)
    # Q = 0: uniform weights over the visible keys, O = prefix mean of V, LSE = ln(count)
    z = torch.zeros_like(q8)
    o, l = _run(z, k8, v8, ds, scale=s, causal=True, out_dtype=F32)
    vr = oracle.dequantize(v8, ds[2])
    want = np.cumsum(vr, axis=2) / np.arange(1, 334)[None, None, :, None]
    assert np.abs(to_f64(o) - want).max() <= 2e-4
    assert np.abs(to_f64(l) - np.log(np.arange(1, 334))[None, None]).max() <= 1e-4


def test_c2_shape_fp8_sampled_rows():
    B, H, N, d = 4, 16, 8192, 128
    print("[case] c2 shape fp8: generating inputs", flush=True)
    q8, k8, v8, ds = W.random_qkv_fp8(B, H, N, d, seed=2)
    g = torch.Generator("cpu").manual_seed(12)
    rows = torch.stack([torch.stack([torch.randperm(N, generator=g)[:256].sort().values for _ in range(H)])
                        for _ in range(B)])
    extra = torch.tensor([0, 1, 127, 128, 255, 256, N - 1])
    rows = torch.cat([rows, extra.expand(B, H, -1)], dim=2)
    print("[case] c2 shape fp8: running", flush=True)
    _check(q8, k8, v8, ds, scale=W.scale_for(d), causal=True, out_dtype=BF16, rows=rows, label="c2-fp8")


def test_fp8_errors_surface():
    q8 = torch.zeros(1, 1, 16, 64, dtype=torch.uint8, device="cuda")
    with pytest.raises(fa.FaUnsupported):
        fa.forward_fp8(torch.zeros(1, 1, 16, 32, dtype=torch.uint8, device="cuda"),
                       torch.zeros(1, 1, 16, 32, dtype=torch.uint8, device="cuda"),
                       torch.zeros(1, 1, 16, 32, dtype=torch.uint8, device="cuda"))
    with pytest.raises(fa.FaInvalidArgument):
        fa.forward_fp8(q8, q8.clone(), q8.clone(), descale_v=float("nan"))


@pytest.mark.parametrize("name", ["c3", "c4"])
def test_workload_shape_fp8_sampled_rows(name):
    """The c3 (key padding, Q/K gain 3) and c4 (N = 131072) shapes at full size with FP8 inputs,
    checked on the workload's seed-chosen rows plus tile-boundary rows."""
    w = W.WORKLOADS[name]
    print(f"[case] {name} fp8: generating inputs", flush=True)
    x = W.make_inputs(w, sample_rows=256)     # seqlens and sampled rows in the documented order
    q8, k8, v8, ds = W.random_qkv_fp8(w.B, w.H, w.N, w.d, w.seed, w.qk_gain)
    mask = w.mask_kinds[0]
    causal = bool(mask & W.MASK_CAUSAL)
    seq = x.seqlens if (mask & W.MASK_KEY_PADDING) else None
    rows = x.rows[:, :, :: max(1, x.rows.shape[-1] // 256)]   # about 256 rows spread over the sorted sample
    extra = torch.tensor([0, 1, 127, 128, w.N - 1])
    rows = torch.cat([rows, extra.expand(w.B, w.H, -1)], dim=2)
    print(f"[case] {name} fp8: running ({rows.shape[-1]} rows per head checked)", flush=True)
    _check(q8, k8, v8, ds, scale=x.scale, causal=causal, seqlens=seq, out_dtype=BF16, rows=rows, label=f"{name}-fp8")


def test_fa_fwd_with_fp8_dtype_equals_unit_descales():
    """fa_fwd with in_dtype FA_DTYPE_FP8_E4M3 is fa_fwd_fp8 with every descale 1 (bitwise)."""
    q8, k8, v8, _ = W.random_qkv_fp8(1, 2, 200, 64, seed=51)
    q, k, v = (t.to("cuda") for t in (q8, k8, v8))
    s = W.scale_for(64)
    o1, l1 = fa.forward_fp8(q, k, v, scale=s, causal=True, out_dtype=F32)
    o2 = torch.empty_like(o1)
    l2 = torch.empty_like(l1)
    stream = torch.cuda.current_stream().cuda_stream
    st = fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o2.data_ptr(), l2.data_ptr(), 1, 2, 200, 64, s,
                   fa.FA_MASK_CAUSAL, None, fa.FA_DTYPE_FP8_E4M3, fa.FA_DTYPE_F32, stream)
    assert st == fa.FA_OK
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fp8_eight_wave_kernel_ragged_n():
    """B*H*ceil(N/256) >= 1024 selects the eight-wave 256-row kernel for causal d = 128; N = 1000
    leaves a ragged last tile (rows 768..999) and a partial diagonal.  Checked on sampled rows
    including every tile boundary."""
    B, H, N, d = 4, 64, 1000, 128
    q8, k8, v8, ds = W.random_qkv_fp8(B, H, N, d, seed=61)
    g = torch.Generator("cpu").manual_seed(62)
    rows = torch.stack([torch.stack([torch.randperm(N, generator=g)[:24].sort().values for _ in range(H)])
                        for _ in range(B)])
    edge = torch.tensor([0, 1, 63, 64, 127, 128, 255, 256, 511, 512, 767, 768, 960, 998, 999])
    rows = torch.cat([rows, edge.expand(B, H, -1)], dim=2)
    _check(q8, k8, v8, ds, scale=W.scale_for(d), causal=True, out_dtype=BF16, rows=rows, label="fp8 eight-wave ragged")


def test_fp8_bitwise_repeatable():
    q8, k8, v8, ds = W.random_qkv_fp8(2, 3, 700, 64, seed=71)
    a = _run(q8, k8, v8, ds, scale=W.scale_for(64), causal=True, out_dtype=BF16)
    b = _run(q8, k8, v8, ds, scale=W.scale_for(64), causal=True, out_dtype=BF16)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [512, 777, 2100])
@pytest.mark.parametrize("mask", list(MASKS))
def test_sweep_fp8_key_split(N, d, mask):
    """Grids small enough for the key split (B*H*ceil(N/32) within its limits, N >= 512): the
    8-bit key-split kernel, every mask, both output types, ragged sizes."""
    causal, pad = MASKS[mask]
    B, H = 1, 2
    q8, k8, v8, ds = W.random_qkv_fp8(B, H, N, d, seed=5000 + N + d)
    seq = None
    if pad:
        g = torch.Generator("cpu").manual_seed(N + 13)
        seq = torch.randint(0, N + 1, (B,), generator=g, dtype=torch.int32)
    for out_dtype in (BF16, F32):
        label = f"key split N={N} d={d} mask={mask} out={out_dtype}"
        print(f"[case] {label}", flush=True)
        _check(q8, k8, v8, ds, scale=W.scale_for(d), causal=causal, seqlens=seq, out_dtype=out_dtype, label=label)
