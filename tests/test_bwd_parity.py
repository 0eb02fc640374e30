"""GPU parity of the backward pass: the HIP kernels through the C ABI against the fp64 oracle.

The forward pass runs on the GPU first (bf16 O and float32 LSE, as a training step would hand
them over); the gradients of the HIP path are compared with ``oracle.attention_bwd_ref`` on the
same bf16 Q, K, V and dO.

Tolerance (per element, derived from the arithmetic of the kernels):
* P and dS enter the value and key products as bf16 values: relative rounding <= 2^-8 each.
* D_i = dO_i . O_i is formed from the bf16 O the forward returned: |dD_i| <= 2^-8 sum_d |dO O|.
* Hence |dV_err| <= 2^-8 |P|^T |dO|, and with e_S = 2^-8 |dS| + P |dD| the errors of dK and dQ
  are at most scale |e_S|^T |Q| and scale |e_S| |K|.  Float32 accumulation and exp2 add far less;
  the test allows twice these bounds plus 1e-5 absolute.
The bounds use the oracle's P and dS (computed here from the fp64 definition, for the bound
only); the expected values themselves come from the oracle alone.
"""

import numpy as np
import pytest
import torch

import exact_tiled_attention_19_amd as fa
import oracle
from exact_tiled_attention_19_amd import workloads as W

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    fa.load_library()


def _f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _bounds(q, k, v, do, o_bf16, scale, causal, seqlens):
    """Per-element error bounds (float64 [B, H, N, d] each) for dQ, dK, dV."""
    q, k, v, do, o = (_f64(t) for t in (q, k, v, do, o_bf16))
    B, H, N, d = q.shape
    u = 2.0 ** -8
    bq, bk, bv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        L = N if seqlens is None else int(min(max(int(seqlens[b]), 0), N))
        for h in range(H):
            P = oracle.softmax_weights_ref(q[b, h], k[b, h], scale, causal=causal, seqlen=L)
            dP = do[b, h] @ v[b, h].T
            D = (P * dP).sum(axis=1)
            dS = P * (dP - D[:, None])
            dD = u * np.abs(do[b, h] * o[b, h]).sum(axis=1)
            eS = u * np.abs(dS) + P * dD[:, None]
            bv[b, h] = u * (np.abs(P).T @ np.abs(do[b, h]))
            bk[b, h] = scale * (eS.T @ np.abs(q[b, h]))
            bq[b, h] = scale * (eS @ np.abs(k[b, h]))
    return bq, bk, bv


def run_case(B, H, N, d, causal, seqlens, seed, label):
    q, k, v, _ = W.random_qkv(B, H, N, d, BF16, seed=seed)
    g = torch.Generator("cpu").manual_seed(seed + 1)
    do = torch.randn(B, H, N, d, generator=g).to(BF16)
    scale = W.scale_for(d)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    sd = None if seqlens is None else torch.tensor(seqlens, dtype=torch.int32, device=DEV)
    o, lse = fa.forward(qd, kd, vd, scale=scale, causal=causal, seqlens=sd, out_dtype=BF16)
    dq, dk, dv = fa.backward(qd, kd, vd, o, lse, dod, scale=scale, causal=causal, seqlens=sd)
    torch.cuda.synchronize()
    got = [_f64(t) for t in (dq, dk, dv)]
    ref = oracle.attention_bwd_ref(q, k, v, do, scale, causal=causal, seqlens=seqlens)
    bounds = _bounds(q, k, v, do, o.cpu(), scale, causal, seqlens)
    worst = {}
    for name, x, r, bd in zip(("dQ", "dK", "dV"), got, ref, bounds):
        assert np.isfinite(x).all(), f"{label}: non-finite {name}"
        err = np.abs(x - r)
        ratio = err / (2.0 * bd + 1e-5)
        worst[name] = (float(err.max()), float(ratio.max()))
        assert ratio.max() <= 1.0, f"{label}: {name} err {err.max():.3e} exceeds the bound (ratio {ratio.max():.3f})"
    print(f"[bwd] {label}: " + ", ".join(f"{n} max_err={e:.3e} ratio={rt:.3f}" for n, (e, rt) in worst.items()),
          flush=True)
    return dq, dk, dv


MASKS = {"none": (False, None), "causal": (True, None), "pad": (False, [37, 300]), "causal_pad": (True, [300, 5])}


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 17, 64, 100, 129, 300])
@pytest.mark.parametrize("mask", list(MASKS))
def test_bwd_sweep(N, d, mask):
    causal, seq = MASKS[mask]
    if seq is not None:
        seq = [min(s, N) for s in seq]
    run_case(2, 2, N, d, causal, seq, seed=3000 + N + d, label=f"N={N} d={d} mask={mask}")


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_memory_budget_shape(causal):
    """The pages' memory-budget shape (one head, N=4096, d=64), in full."""
    run_case(1, 1, 4096, 64, causal, None, seed=41, label=f"N=4096 d=64 causal={causal}")


def test_bwd_long_causal_d128():
    run_case(1, 2, 2048, 128, True, None, seed=42, label="B=1 H=2 N=2048 d=128 causal")


def test_bwd_all_masked_rows_and_determinism():
    """Valid length 0: every gradient is exactly 0 (no NaN); two runs agree bitwise."""
    B, H, N, d = 2, 1, 96, 64
    q, k, v, _ = W.random_qkv(B, H, N, d, BF16, seed=5)
    do = torch.randn(B, H, N, d, generator=torch.Generator("cpu").manual_seed(6)).to(BF16)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    sd = torch.tensor([0, 50], dtype=torch.int32, device=DEV)
    o, lse = fa.forward(qd, kd, vd, seqlens=sd, out_dtype=BF16)
    a = fa.backward(qd, kd, vd, o, lse, dod, seqlens=sd)
    b = fa.backward(qd, kd, vd, o, lse, dod, seqlens=sd)
    torch.cuda.synchronize()
    for x in a:
        assert torch.isfinite(x).all()
        assert torch.count_nonzero(x[0]) == 0
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    # keys past the valid length of batch element 1 get no gradient
    assert torch.count_nonzero(a[1][1, :, 50:]) == 0 and torch.count_nonzero(a[2][1, :, 50:]) == 0


def test_bwd_errors_surface():
    x = torch.zeros(1, 1, 16, 64, dtype=BF16, device=DEV)
    lse = torch.zeros(1, 1, 16, dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError):
        fa.backward(x, x, x, x, lse, x.float())
    # a gradient output overlapping an input is rejected by the library
    g = torch.zeros(1, 1, 16, 64, dtype=torch.float32, device=DEV)
    with pytest.raises(fa.FaInvalidArgument):
        fa.backward(x, x, x, x, lse, x, out=(g, g, torch.zeros_like(g)))
