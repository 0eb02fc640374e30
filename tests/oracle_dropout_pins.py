"""Pins of the dropout oracle: the published Philox known answers, the contract's structure, and
what the mathematics fixes.

Each pin takes an ``impl`` namespace (the oracle package, or a mutant of the dropout module)
and raises on a mismatch.

* Philox4x32-10 reproduces the known-answer vectors published with the generator
  (tests/golden/philox_kat.json), and the vectorised generator equals the scalar one.
* The contract maps every (row, key) pair to its own byte (no two share one), and the kept
  fraction and byte histogram match a uniform generator.
* p = 0 drops nothing: the output equals the pinned attention oracle; the log-sum-exp never
  depends on dropout.
* Averaged over many seeds the dropped-out output is unbiased.
* A brute-force evaluation with the contract's mask written out.
* The gradient equals central differences of the dropout forward with the mask held fixed.
"""

from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand(seed, B=1, H=2, N=9, d=4):
    g = np.random.default_rng(seed)
    return (g.standard_normal((B, H, N, d)), g.standard_normal((B, H, N, d)), g.standard_normal((B, H, N, d)))


def pin_philox_known_answers(impl):
    with open(os.path.join(GOLDEN, "philox_kat.json")) as f:
        kat = json.load(f)["philox4x32_10"]
    for case in kat:
        c = [int(x, 16) for x in case["counter"]]
        k = [int(x, 16) for x in case["key"]]
        want = tuple(int(x, 16) for x in case["out"])
        got = impl.philox4x32(c, k, 10)
        assert tuple(got) == want, (case, [hex(x) for x in got])
        got_np = impl._philox_np(*[np.array([x], dtype=np.uint64) for x in c], k[0], k[1])
        assert tuple(int(w[0]) for w in got_np) == want


def pin_mask_matches_scalar_contract(impl):
    """The vectorised mask equals the element-by-element evaluation with the scalar generator."""
    for bh, seed, off, p in ((0, 0, 0, 0.3), (5, 0x123456789ABCDEF, 7, 0.1), (2, 2 ** 63 + 11, 2 ** 32 - 1, 0.75)):
        a = impl.keep_mask(bh, 13, 10, seed, off, p)
        b = impl.keep_mask_loop(bh, 13, 10, seed, off, p)
        assert np.array_equal(a, b), (bh, seed, off, p)


def pin_mask_statistics(impl):
    """Kept fraction within 5 sigma of 1 - t/256 on 256 x 256 draws, for several p, and the
    masks of different heads, offsets and seeds are different."""
    n = 256
    for p in (0.1, 0.5, 0.9):
        t = impl.dropout_threshold(p)
        m = impl.keep_mask(3, n, n, 1234, 5, p)
        q = 1 - t / 256
        sd = np.sqrt(q * (1 - q) / m.size)
        assert abs(m.mean() - q) < 5 * sd, (p, m.mean(), q)
    base = impl.keep_mask(3, 64, 64, 1234, 5, 0.5)
    for other in (impl.keep_mask(4, 64, 64, 1234, 5, 0.5), impl.keep_mask(3, 64, 64, 1234, 6, 0.5),
                  impl.keep_mask(3, 64, 64, 1235, 5, 0.5)):
        assert 0.4 < (base != other).mean() < 0.6
    # rows and columns are not tied: the keep decisions of (i, j) and (j, i) agree half the time
    assert 0.4 < (base == base.T).mean() < 0.6


def pin_threshold(impl):
    assert impl.dropout_threshold(0.0) == 0 and impl.dropout_threshold(0.5) == 128
    assert impl.dropout_threshold(0.1) == 26 and impl.dropout_threshold(255 / 256) == 255
    for bad in (-0.01, 1.0):
        try:
            impl.dropout_threshold(bad)
        except ValueError:
            continue
        raise AssertionError(f"p={bad} accepted")


def pin_p_zero_is_attention(impl):
    q, k, v = _rand(1)
    for causal, seq in ((False, None), (True, None), (False, [5])):
        O, L = impl.attention_dropout_ref(q, k, v, 0.6, 0.0, 99, 3, causal=causal, seqlens=seq)
        Or, Lr = impl.attention_ref(q, k, v, 0.6, causal=causal, seqlens=seq)
        assert np.allclose(O, Or, atol=1e-14) and np.array_equal(L, Lr)


def pin_lse_ignores_dropout(impl):
    q, k, v = _rand(2)
    _, L = impl.attention_dropout_ref(q, k, v, 0.6, 0.4, 99, 3, causal=True)
    _, Lr = impl.attention_ref(q, k, v, 0.6, causal=True)
    assert np.array_equal(L, Lr)


def pin_unbiased(impl):
    """The mean over 400 seeds approaches the undropped output (5 sigma per element)."""
    q, k, v = _rand(3, N=6, d=3)
    Or, _ = impl.attention_ref(q, k, v, 0.8, causal=True)
    outs = np.stack([impl.attention_dropout_ref(q, k, v, 0.8, 0.3, s, 0, causal=True)[0] for s in range(400)])
    mean, sd = outs.mean(axis=0), outs.std(axis=0) / np.sqrt(len(outs))
    assert np.all(np.abs(mean - Or) <= 5 * sd + 1e-12), np.max(np.abs(mean - Or) / (sd + 1e-30))


def pin_brute_force(impl):
    """Pure-Python loops over the definition O_i = sum_j P_ij Z_ij v_j with the contract's mask."""
    import math
    q, k, v = _rand(4, B=1, H=1, N=7, d=3)
    p, seed, off, c = 0.25, 0xDEADBEEF12345678, 9, 0.7
    O, _ = impl.attention_dropout_ref(q, k, v, c, p, seed, off, causal=True)
    t = impl.dropout_threshold(p)
    for i in range(7):
        s = [c * math.fsum(q[0, 0, i, e] * k[0, 0, j, e] for e in range(3)) for j in range(i + 1)]
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        den = math.fsum(w)
        for e in range(3):
            acc = []
            for j in range(i + 1):
                words = impl.philox4x32((j // 4, i // 4, 0, off), (seed, seed >> 32), 10)
                kept = ((words[i % 4] >> (8 * (j % 4))) & 0xFF) >= t
                acc.append(w[j] / den * (256 / (256 - t) if kept else 0.0) * v[0, 0, j, e])
            assert abs(O[0, 0, i, e] - math.fsum(acc)) < 1e-13


def pin_gradient_finite_differences(impl):
    """Central differences of L = sum(O * G) through the dropout forward (mask fixed by the seed)."""
    h = 1e-5
    q, k, v = _rand(5, B=1, H=1, N=6, d=3)
    G = np.random.default_rng(6).standard_normal(q.shape)
    for causal, seq in ((False, None), (True, None), (False, [4])):
        dq, dk, dv = impl.attention_dropout_bwd_ref(q, k, v, G, 0.7, 0.3, 17, 2, causal=causal, seqlens=seq)
        for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                args = {"q": q, "k": k, "v": v}
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args[name] = xp
                fp = (impl.attention_dropout_ref(args["q"], args["k"], args["v"], 0.7, 0.3, 17, 2, causal=causal,
                                                 seqlens=seq)[0] * G).sum()
                args[name] = xm
                fm = (impl.attention_dropout_ref(args["q"], args["k"], args["v"], 0.7, 0.3, 17, 2, causal=causal,
                                                 seqlens=seq)[0] * G).sum()
                num[idx] = (fp - fm) / (2 * h)
            assert np.abs(num - grad).max() < 1e-7, (name, causal, seq, np.abs(num - grad).max())


PINS = [pin_philox_known_answers, pin_mask_matches_scalar_contract, pin_mask_statistics, pin_threshold,
        pin_p_zero_is_attention, pin_lse_ignores_dropout, pin_unbiased, pin_brute_force,
        pin_gradient_finite_differences]
