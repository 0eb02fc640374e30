"""The pipelined kernel's exponent-shift rule, replayed on the CPU in float32 (no GPU).

With a bf16 output the pipelined forward (csrc/fa_fwd_bf16_pipe.h) keeps, per query row, a
shift m (log2 units), a running sum l of 2^(s*c - m) and an unnormalised accumulator, updated one
64-key tile at a time as in "FlashAttention Interview Questions: IO Complexity, Tiling, and
Numerical Stability", section "How can softmax be computed across tiles?".  To save rescales it
may leave a rise of the row maximum unapplied; then the tile's probabilities exceed 1.  The page's
section "Does subtracting the maximum solve every numerical issue?" explains that the shift is
what keeps the exponentials from overflowing, so any rule that lags behind the maximum must still
bound them.

``replay_row`` follows the kernel's order of operations for one row, in float32:

* the first tile's maximum always becomes the shift (the prologue tracks the exact maximum);
* for each later tile, the decision uses the row sum over every earlier tile (the kernel adds
  tile j's sum in phase A and decides for tile j+1 in phase B);
* a taken rise multiplies l and the accumulator by 2^(m_old - m_new);
* p = 2^(s*c - m) is summed in float32 and enters the value product as a bf16 value.

Two rules are replayed: the one without a cap (skip while 2^rise * 4 <= l), and the kernel's
rule, which also moves the shift whenever the rise exceeds 8.  On logits that climb steadily
along the keys, the uncapped rule lets the shift fall ever further behind, l overflows float32
and O becomes NaN; the capped rule keeps every probability <= 2^8 and matches the fp64 oracle.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_19_amd import workloads as W

F32 = np.float32
SKIP_CAP = 8.0    # the kernel's kSkipCap (log2 units)
TILE = 64         # keys per tile of the pipelined kernel


def _bf16(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=F32)).to(torch.bfloat16).float().numpy()


def replay_row(s_raw: np.ndarray, v: np.ndarray, c: float, capped: bool, wmul: float = 4.0):
    """One query row through the kernel's online update in float32.

    s_raw: float32 dot products q . k_j of the row's visible keys (unscaled); v: [n, d] values;
    c: scale * log2(e) as float32.  Returns (O, l, m, largest p entering the value product).
    """
    c = F32(c)
    m = F32(-np.inf)
    l = F32(0.0)
    acc = np.zeros(v.shape[1], dtype=F32)
    p_max = 0.0
    with np.errstate(over="ignore", invalid="ignore"):
        for t0 in range(0, len(s_raw), TILE):
            s = s_raw[t0:t0 + TILE].astype(F32)
            m_tile = F32(s.max() * c)
            if m == -np.inf:
                need = True
            else:
                rise = F32(m_tile - m)
                over = F32(np.exp2(rise)) * F32(wmul) > l
                need = bool(rise > 0 and ((capped and rise > SKIP_CAP) or over))
            if need:
                alpha = F32(np.exp2(F32(m - m_tile))) if m != -np.inf else F32(0.0)
                m = m_tile
                l = F32(l * alpha)
                acc = (acc * alpha).astype(F32)
            p = np.exp2((s * c - m).astype(F32)).astype(F32)
            p_max = max(p_max, float(p.max()))
            l = F32(l + p.sum(dtype=F32))
            acc = (acc + _bf16(p) @ v[t0:t0 + TILE].astype(F32)).astype(F32)
        return (acc / l).astype(F32), float(l), float(m), p_max


def _ramp_row(n: int, d: int, span: float, seed: int):
    """Row n-1 of W.ramp_qkv's non-causal head: every key visible, logits climbing to ``span``."""
    q, k, v = W.ramp_qkv(1, 1, n, d, span, torch.bfloat16, seed)
    qf, kf, vf = (x.float().numpy()[0, 0] for x in (q, k, v))
    s = (kf @ qf[n - 1]).astype(F32)       # float32 dot products, as the MFMA accumulates them
    return q, k, v, s, vf


@pytest.mark.parametrize("n,span", [(4096, 110.0), (8192, 110.0), (13000, 95.0)])
def test_uncapped_rule_overflows_on_a_climbing_row(n, span):
    d = 128
    c = F32(W.scale_for(d) * math.log2(math.e))
    _, _, _, s, vf = _ramp_row(n, d, span, seed=1)
    O, l, m, p_max = replay_row(s, vf, c, capped=False)
    # the shift stays near the first tile's maximum while the row climbs by ~span nats
    assert not math.isfinite(l) and not np.isfinite(O).all(), (l, m, p_max)


@pytest.mark.parametrize("n,span", [(4096, 110.0), (8192, 110.0), (13000, 95.0)])
def test_capped_rule_matches_the_oracle_on_a_climbing_row(n, span):
    d = 128
    scale = W.scale_for(d)
    c = F32(scale * math.log2(math.e))
    q, k, v, s, vf = _ramp_row(n, d, span, seed=1)
    O, l, m, p_max = replay_row(s, vf, c, capped=True)
    assert p_max <= 2.0 ** SKIP_CAP and l <= 2.0 ** SKIP_CAP * n
    O_ref, _ = oracle.attention_ref(q, k, v, scale, rows=[n - 1])
    # bf16-output tolerance of the forward (per element max(1e-2, half a bf16 ulp + 1e-3))
    err = float(np.abs(O.astype(np.float64) - O_ref[0, 0, 0]).max())
    assert err <= 1e-2, err


def test_capped_rule_bounds_every_probability_on_random_and_peaked_rows():
    """Rows of every shape the workloads produce (flat, peaked x3, climbing, falling): the largest
    probability that enters the value product is <= 2^8 and O matches the oracle."""
    d, n = 64, 3000
    scale = W.scale_for(d)
    c = F32(scale * math.log2(math.e))
    for gain, seed in ((1.0, 3), (3.0, 4)):
        q, k, v, _ = W.random_qkv(1, 1, n, d, torch.bfloat16, seed, qk_gain=gain)
        qf, kf, vf = (x.float().numpy()[0, 0] for x in (q, k, v))
        rows = [0, 1, 700, n - 1]
        O_ref, _ = oracle.attention_ref(q, k, v, scale, rows=rows)
        for r, i in enumerate(rows):
            s = (kf @ qf[i]).astype(F32)
            for order in (slice(None), slice(None, None, -1)):
                if order.step == -1:   # keys reversed: the oracle result is permutation invariant
                    O, _, _, p_max = replay_row(s[order], vf[order], c, capped=True)
                else:
                    O, _, _, p_max = replay_row(s, vf, c, capped=True)
                assert p_max <= 2.0 ** SKIP_CAP
                assert float(np.abs(O - O_ref[0, 0, r]).max()) <= 1e-2


def test_replay_agrees_with_the_exact_shift_when_nothing_is_skipped():
    """Control: on the pages' two-key example (one tile), the replay is the plain online update:
    output 5 for values 2 and 6 with weights 1/4 and 3/4."""
    s = np.array([0.0, math.log(3.0)], dtype=F32)
    v = np.array([[2.0], [6.0]], dtype=F32)
    c = F32(math.log2(math.e))
    O, l, m, _ = replay_row(s, v, c, capped=True)
    assert abs(float(O[0]) - 5.0) < 2e-2 and abs(l - 4.0 / 3.0) < 1e-6
