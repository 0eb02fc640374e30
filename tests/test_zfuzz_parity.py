"""GPU parity on seeded random shapes: every entry point against its fp64 oracle at sizes and
combinations the hand-written cases do not list (odd lengths, mixed masks, kernel variants,
packed batches with empty and over-full sequences, dropout probabilities and seeds).

Each case prints its parameters before it runs.  Tolerances are those of the dedicated tests:
the forward's (float32 out 2e-4 / LSE 1e-4; bf16 out per element max(1e-2, half ulp + 1e-3))
and, for the backward, the per-element bound derived in tests/test_bwd_parity.py.
"""

import numpy as np
import pytest
import torch

import exact_tiled_attention_19_amd as fa
import oracle
from exact_tiled_attention_19_amd import workloads as W
from tests import parity_util as PU

pytestmark = pytest.mark.gpu

BF16, F32 = torch.bfloat16, torch.float32
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    fa.load_library()


def _draw(seed):
    return np.random.default_rng(seed)


@pytest.mark.parametrize("case", range(24))
def test_fuzz_forward(case):
    r = _draw(9000 + case)
    B, H, N = int(r.integers(1, 4)), int(r.integers(1, 4)), int(r.integers(1, 700))
    d = int(r.choice([64, 128]))
    causal = bool(r.integers(0, 2))
    pad = bool(r.integers(0, 2))
    out_dtype = BF16 if r.integers(0, 2) else F32
    variants = [0, 1, 2] + ([3] if d == 128 else [])
    variant = int(r.choice(variants))
    gain = float(r.choice([1.0, 3.0]))
    label = f"forward B={B} H={H} N={N} d={d} causal={causal} pad={pad} out={out_dtype} variant={variant} gain={gain}"
    print(f"[fuzz] {label}", flush=True)
    q, k, v, g = W.random_qkv(B, H, N, d, BF16, seed=9100 + case, qk_gain=gain)
    seq = torch.tensor(r.integers(0, N + 1, B), dtype=torch.int32) if pad else None
    PU.check_case(q, k, v, scale=W.scale_for(d), causal=causal, seqlens=seq, out_dtype=out_dtype, variant=variant,
                  label=label)


@pytest.mark.parametrize("case", range(16))
def test_fuzz_varlen(case):
    r = _draw(9200 + case)
    nseq = int(r.integers(1, 6))
    decode = bool(r.integers(0, 2))
    lq = [int(x) for x in (r.integers(0, 5, nseq) if decode else r.integers(0, 400, nseq))]
    lk = [int(x) for x in r.integers(0, 1200, nseq)]
    if max(lq) == 0:
        lq[0] = 1
    H, d = int(r.integers(1, 4)), int(r.choice([64, 128]))
    causal = bool(r.integers(0, 2))
    align = str(r.choice(["bottom_right", "top_left"]))
    out_dtype = BF16 if r.integers(0, 2) else F32
    label = f"varlen lq={lq} lk={lk} H={H} d={d} causal={causal} align={align} out={out_dtype}"
    print(f"[fuzz] {label}", flush=True)
    q, k, v, cu_q, cu_k = W.random_packed(lq, lk, H, d, BF16, seed=9300 + case)
    scale = W.scale_for(d)
    o, lse = fa.forward_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cu_q.to(DEV), cu_k.to(DEV), max(lq), max(lk),
                               scale=scale, causal=causal, align=align, out_dtype=out_dtype)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention_varlen_ref(q, k, v, cu_q.tolist(), cu_k.tolist(), scale, causal=causal, align=align)
    PU.compare(o.cpu(), lse.cpu(), O_ref, L_ref, out_dtype, label=label)


@pytest.mark.parametrize("case", range(12))
def test_fuzz_dropout_forward(case):
    r = _draw(9400 + case)
    B, H, N = int(r.integers(1, 3)), int(r.integers(1, 3)), int(r.integers(1, 500))
    d = int(r.choice([64, 128]))
    causal, pad = bool(r.integers(0, 2)), bool(r.integers(0, 2))
    p = float(r.integers(0, 230)) / 256.0
    seed, off = int(r.integers(0, 2 ** 63)), int(r.integers(0, 2 ** 32))
    label = f"dropout B={B} H={H} N={N} d={d} causal={causal} pad={pad} p={p:.4f} seed={seed} offset={off}"
    print(f"[fuzz] {label}", flush=True)
    q, k, v, _ = W.random_qkv(B, H, N, d, BF16, seed=9500 + case)
    seq = [int(x) for x in r.integers(0, N + 1, B)] if pad else None
    sd = None if seq is None else torch.tensor(seq, dtype=torch.int32, device=DEV)
    o, lse = fa.forward_dropout(q.to(DEV), k.to(DEV), v.to(DEV), p, seed, off, scale=W.scale_for(d), causal=causal,
                                seqlens=sd, out_dtype=F32)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention_dropout_ref(q, k, v, W.scale_for(d), p, seed, off, causal=causal, seqlens=seq)
    PU.compare(o.cpu(), lse.cpu(), O_ref, L_ref, F32, label=label)


@pytest.mark.parametrize("case", range(8))
def test_fuzz_backward(case):
    from tests.test_bwd_parity import run_case
    r = _draw(9600 + case)
    B, H, N = int(r.integers(1, 3)), int(r.integers(1, 3)), int(r.integers(1, 400))
    d = int(r.choice([64, 128]))
    causal, pad = bool(r.integers(0, 2)), bool(r.integers(0, 2))
    seq = [int(x) for x in r.integers(0, N + 1, B)] if pad else None
    print(f"[fuzz] backward B={B} H={H} N={N} d={d} causal={causal} seqlens={seq}", flush=True)
    run_case(B, H, N, d, causal, seq, seed=9700 + case, label=f"fuzz backward case {case}")
