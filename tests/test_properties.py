"""GPU property tests: invariants and closed forms checked directly on the HIP path.

Sources: "FlashAttention Interview Questions: IO Complexity, Tiling, and Numerical Stability"
(cswork.org) -- shift invariance and the +1,000 exercise, masked tiles add no mass, an all-masked
row needs a defined result, extreme values at masked positions change nothing, a late tile with
a much larger maximum exercises the rescaling, exact target (section "What is FlashAttention
exact about?").  The tests also check run-to-run determinism, stream ordering and that the
library allocates no device memory.
"""

import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_19_amd as fa
from exact_tiled_attention_19_amd import workloads as W
from tests.parity_util import TOL_LSE, TOL_O_F32, check_case, to_f64

pytestmark = pytest.mark.gpu

BF16, F32 = torch.bfloat16, torch.float32
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    fa.load_library()


def run(q, k, v, **kw):
    o, lse = fa.forward(q.to(DEV), k.to(DEV), v.to(DEV), **kw)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("pad", [False, True])
def test_q_zero_gives_mean_of_visible_values(d, causal, pad):
    """Q = 0: every visible score is 0, so O_i is the mean of the visible V rows and
    LSE_i = ln(count); P = 1 exactly, so the float32 output is tight."""
    B, H, N = 2, 2, 300
    _, k, v, _ = W.random_qkv(B, H, N, d, BF16, seed=3)
    q = torch.zeros_like(k)
    seq = torch.tensor([N, 137], dtype=torch.int32) if pad else None
    o, lse = run(q, k, v, causal=causal, seqlens=None if seq is None else seq.to(DEV), out_dtype=F32)
    vv = to_f64(v)
    for b in range(B):
        L = N if seq is None else int(seq[b])
        cnt = np.minimum(np.arange(1, N + 1), L) if causal else np.full(N, L)
        csum = np.cumsum(vv[b, :, :L], axis=1)
        want = csum[:, cnt - 1] / cnt[None, :, None]
        assert np.abs(to_f64(o[b]) - want).max() < 1e-5
        assert np.abs(to_f64(lse[b]) - np.log(cnt)[None]).max() < 2e-6


@pytest.mark.parametrize("out_dtype", [BF16, F32])
def test_all_ones_values_give_ones(out_dtype):
    q, k, _, _ = W.random_qkv(1, 4, 517, 128, BF16, seed=4)
    v = torch.ones_like(q)
    o, _ = run(q, k, v, causal=True, out_dtype=out_dtype)
    tol = 8e-3 if out_dtype == BF16 else 2e-5
    assert (to_f64(o) - 1.0).__abs__().max() < tol


def test_constant_channel_shift():
    """Overwriting channel 0 with q = alpha, k = beta adds alpha*beta*scale to every score:
    O is unchanged and LSE moves by exactly that amount (softmax shift invariance; the
    cswork.org page's +1,000 exercise in kernel form)."""
    B, H, N, d = 1, 2, 400, 64
    q, k, v, _ = W.random_qkv(B, H, N, d, BF16, seed=6)
    scale = W.scale_for(d)
    q0, k0 = q.clone(), k.clone()
    q0[..., 0] = 0
    k0[..., 0] = 0
    alpha, beta = 8.0, 10.0         # exact in bf16; alpha*beta*scale = 10
    q1, k1 = q0.clone(), k0.clone()
    q1[..., 0] = alpha
    k1[..., 0] = beta
    for causal in (False, True):
        oa, la = run(q0, k0, v, causal=causal, out_dtype=F32)
        ob, lb = run(q1, k1, v, causal=causal, out_dtype=F32)
        assert (to_f64(oa) - to_f64(ob)).__abs__().max() < 5e-5
        shift = alpha * beta * scale
        assert np.abs(to_f64(lb) - to_f64(la) - shift).max() < 2e-4


def test_key_value_permutation():
    B, H, N, d = 1, 2, 640, 128
    q, k, v, _ = W.random_qkv(B, H, N, d, BF16, seed=8)
    p = torch.randperm(N, generator=torch.Generator().manual_seed(1))
    oa, la = run(q, k, v, out_dtype=F32)
    ob, lb = run(q, k[:, :, p].contiguous(), v[:, :, p].contiguous(), out_dtype=F32)
    assert (to_f64(oa) - to_f64(ob)).__abs__().max() < 2 * TOL_O_F32
    assert (to_f64(la) - to_f64(lb)).__abs__().max() < TOL_LSE


@pytest.mark.parametrize("out_dtype", [BF16, F32])
def test_masked_extremes_change_nothing(out_dtype):
    """Extreme finite values at masked K/V positions leave every output bit unchanged."""
    B, H, N, d = 2, 2, 333, 128
    q, k, v, _ = W.random_qkv(B, H, N, d, BF16, seed=10)
    seq = torch.tensor([200, 65], dtype=torch.int32)
    o1, l1 = run(q, k, v, seqlens=seq.to(DEV), out_dtype=out_dtype)
    k2, v2 = k.clone(), v.clone()
    for b in range(B):
        L = int(seq[b])
        k2[b, :, L:] = 3.0e38
        k2[b, :, L:, ::2] = -3.0e38
        v2[b, :, L:] = -3.0e38
    o2, l2 = run(q, k2, v2, seqlens=seq.to(DEV), out_dtype=out_dtype)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # causal: keys >= j0 extreme; query rows < j0 must not change at all
    j0 = 150
    o3, l3 = run(q, k, v, causal=True, out_dtype=out_dtype)
    k4, v4 = k.clone(), v.clone()
    k4[:, :, j0:] = 1.0e4
    v4[:, :, j0:] = -3.0e38
    o4, l4 = run(q, k4, v4, causal=True, out_dtype=out_dtype)
    assert torch.equal(o3[:, :, :j0], o4[:, :, :j0]) and torch.equal(l3[:, :, :j0], l4[:, :, :j0])


def test_late_tile_with_much_larger_maximum():
    """K_j = c_j u with c_j increasing along the sequence and every query parallel to u: each
    new key tile raises the row maximum, so every tile exercises the rescaling."""
    B, H, N, d = 1, 2, 700, 64
    g = torch.Generator().manual_seed(12)
    u = torch.randn(d, generator=g)
    u = u / u.norm()
    c = torch.linspace(0.0, 12.0, N)
    k = (c[:, None] * u[None, :]).expand(B, H, N, d).clone() + 0.05 * torch.randn(B, H, N, d, generator=g)
    q = (2.0 * u).expand(B, H, N, d).clone() + 0.05 * torch.randn(B, H, N, d, generator=g)
    v = torch.randn(B, H, N, d, generator=g)
    q, k, v = q.to(BF16), k.to(BF16), v.to(BF16)
    for causal in (False, True):
        for out_dtype in (F32, BF16):
            check_case(q, k, v, scale=1.0, causal=causal, out_dtype=out_dtype, label=f"late-max causal={causal}")


def test_pages_two_tile_example_on_gpu():
    """The cswork.org two-tile example inside a head: query 0 = (1, 0, ..), keys (0, ..) and
    (ln 3, ..) with values 2 and 6 -> output 5, LSE ln 4; shifted by +1000 -> still 5."""
    d = 64
    for shift in (0.0, 1000.0):
        q = torch.zeros(1, 1, 2, d)
        k = torch.zeros(1, 1, 2, d)
        v = torch.zeros(1, 1, 2, d)
        q[0, 0, 0, 0] = 1.0
        q[0, 0, 0, 1] = shift
        k[0, 0, 0, 0] = 0.0
        k[0, 0, 1, 0] = math.log(3.0)
        k[0, 0, :, 1] = 1.0
        v[0, 0, 0, 0] = 2.0
        v[0, 0, 1, 0] = 6.0
        # bf16 rounds ln 3; use float32 inputs so the example is exact to float32
        o, lse = run(q, k, v, scale=1.0, out_dtype=F32)
        # float32 scores near 1000 carry an ulp of 2^-14, so the shifted case gets a looser bound
        assert abs(float(o[0, 0, 0, 0]) - 5.0) < (1e-5 if shift == 0 else 1e-4)
        assert abs(float(lse[0, 0, 0]) - (shift + math.log(4.0))) < (1e-5 if shift == 0 else 1e-3)


def test_all_masked_rows():
    """seqlens 0 (and negative, clamped to 0): O = 0 and LSE = -inf, never NaN; seqlens above N
    are clamped to N."""
    B, H, N, d = 3, 2, 200, 64
    q, k, v, _ = W.random_qkv(B, H, N, d, BF16, seed=14)
    seq = torch.tensor([0, -5, 10 * N], dtype=torch.int32)
    for causal in (False, True):
        for out_dtype in (BF16, F32):
            o, lse = run(q, k, v, causal=causal, seqlens=seq.to(DEV), out_dtype=out_dtype)
            assert torch.all(o[:2] == 0) and torch.all(torch.isneginf(lse[:2]))
            o_full, lse_full = run(q[2:], k[2:], v[2:], causal=causal, out_dtype=out_dtype)
            assert torch.equal(o[2:], o_full) and torch.equal(lse[2:], lse_full)
    # float32 path too
    qf, kf, vf = q.float(), k.float(), v.float()
    o, lse = run(qf, kf, vf, seqlens=seq.to(DEV))
    assert torch.all(o[:2] == 0) and torch.all(torch.isneginf(lse[:2]))


def test_deterministic_bitwise():
    q, k, v, _ = W.random_qkv(2, 4, 1111, 128, BF16, seed=15)
    a = run(q, k, v, causal=True)
    b = run(q, k, v, causal=True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_no_lse_pointer_and_side_stream():
    """LSE may be omitted; work is ordered on the caller's stream (a non-default stream)."""
    q, k, v, _ = W.random_qkv(1, 2, 257, 64, BF16, seed=16)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    ref, _ = fa.forward(qd, kd, vd, causal=True)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, lse = fa.forward(qd, kd, vd, causal=True, return_lse=False)
    s.synchronize()
    assert lse is None and torch.equal(o, ref)


def test_library_allocates_nothing():
    """With outputs preallocated, a call changes neither torch's allocation counters nor the
    device's free memory: there is no N x N (or any) workspace."""
    q, k, v, _ = W.random_qkv(1, 8, 4096, 128, BF16, seed=17)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o = torch.empty_like(qd)
    lse = torch.empty(1, 8, 4096, dtype=torch.float32, device=DEV)
    fa.forward(qd, kd, vd, causal=True, out=o, lse_out=lse)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    alloc0 = torch.cuda.memory_allocated()
    for _ in range(3):
        fa.forward(qd, kd, vd, causal=True, out=o, lse_out=lse)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert torch.cuda.memory_allocated() == alloc0
    assert free1 == free0


def test_errors_surface_as_exceptions():
    q, k, v, _ = W.random_qkv(1, 1, 16, 96, BF16, seed=18)
    with pytest.raises(fa.FaUnsupported):
        fa.forward(q.to(DEV), k.to(DEV), v.to(DEV))
    q, k, v, _ = W.random_qkv(1, 1, 16, 64, BF16, seed=18)
    with pytest.raises(fa.FaInvalidArgument):
        fa.forward(q.to(DEV), k.to(DEV), v.to(DEV), scale=float("nan"))
