"""GPU parity of the forward with dropout (fa_fwd_dropout) against the fp64 dropout oracle.

Both sides draw the mask from the contract of include/fa.h (Philox4x32-10 per 4 x 4 block of
(row, key) pairs, byte threshold round(256 p)); the HIP kernels generate it on the device and the
oracle in numpy, with no shared code.  With a float32 output every element of O is checked to
2e-4 at sizes where a single wrongly kept or dropped probability would move O by far more
(about keep_scale * |v| / N), so the comparison also proves the kernel's mask bit for bit; with a
bf16 output the forward's per-element bound applies.  The LSE is that of the undropped
probabilities and must equal fa_fwd's bit for bit.
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
F32 = torch.float32
DEV = "cuda"
MASKS = {"none": (False, None), "causal": (True, None), "pad": (False, [37, 300]), "causal_pad": (True, [300, 5])}


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    fa.load_library()


def run(B, H, N, d, causal, seq, p, seed, offset, out_dtype, data_seed, label):
    q, k, v, _ = W.random_qkv(B, H, N, d, BF16, seed=data_seed)
    scale = W.scale_for(d)
    sd = None if seq is None else torch.tensor(seq, dtype=torch.int32, device=DEV)
    print(f"[dropout] {label}", flush=True)
    o, lse = fa.forward_dropout(q.to(DEV), k.to(DEV), v.to(DEV), p, seed, offset, scale=scale, causal=causal,
                                seqlens=sd, out_dtype=out_dtype)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention_dropout_ref(q, k, v, scale, p, seed, offset, causal=causal, seqlens=seq)
    res = PU.compare(o.cpu(), lse.cpu(), O_ref, L_ref, out_dtype, label=label)
    print(f"[dropout] {label}: {res}", flush=True)
    return q, k, v, o, lse


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 17, 100, 129, 300])
@pytest.mark.parametrize("mask", list(MASKS))
def test_dropout_sweep_f32(N, d, mask):
    causal, seq = MASKS[mask]
    if seq is not None:
        seq = [min(s, N) for s in seq]
    run(2, 2, N, d, causal, seq, 0.2, 0x5EED0000 + N, 3, F32, 4000 + N + d, f"N={N} d={d} mask={mask} p=0.2")


@pytest.mark.parametrize("p", [0.05, 0.5, 0.9])
@pytest.mark.parametrize("out_dtype", [BF16, F32], ids=["bf16", "f32"])
def test_dropout_probabilities(p, out_dtype):
    run(1, 3, 260, 128, True, None, p, 2 ** 63 + 12345, 7, out_dtype, 4100, f"p={p} out={out_dtype}")


def test_dropout_longer_rows():
    """Rows of up to 1536 keys, several pipeline iterations per tile, seed words with high bits."""
    run(1, 2, 1536, 64, True, None, 0.1, 0xFFFFFFFF00000001, 2 ** 32 - 1, F32, 4200, "N=1536 d=64 causal p=0.1")


def test_dropout_reproducible_and_lse_unchanged():
    """Same (seed, offset): bitwise the same output; another offset or seed: another mask; the LSE
    equals fa_fwd's bit for bit; p = 0 gives fa_fwd's output bit for bit."""
    q, k, v, _ = W.random_qkv(2, 2, 200, 128, BF16, seed=4300)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    a = fa.forward_dropout(qd, kd, vd, 0.3, 99, 1, causal=True, out_dtype=F32)
    b = fa.forward_dropout(qd, kd, vd, 0.3, 99, 1, causal=True, out_dtype=F32)
    c = fa.forward_dropout(qd, kd, vd, 0.3, 99, 2, causal=True, out_dtype=F32)
    e = fa.forward_dropout(qd, kd, vd, 0.3, 100, 1, causal=True, out_dtype=F32)
    z = fa.forward_dropout(qd, kd, vd, 0.0, 99, 1, causal=True, out_dtype=F32)
    r = fa.forward(qd, kd, vd, causal=True, out_dtype=F32)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert not torch.equal(a[0], c[0]) and not torch.equal(a[0], e[0])
    assert torch.equal(a[1], r[1]) and torch.equal(c[1], r[1])
    assert torch.equal(z[0], r[0])


def test_dropout_errors_surface():
    x = torch.zeros(1, 1, 16, 64, dtype=BF16, device=DEV)
    with pytest.raises(fa.FaInvalidArgument):
        fa.forward_dropout(x, x, x, 1.0, 0)
    with pytest.raises(ValueError):
        fa.forward_dropout(x.float(), x.float(), x.float(), 0.1, 0)
