"""Pins of the fp64 packed variable-length oracle: what the pages and the mathematics fix.

Each pin takes an ``impl`` namespace (the oracle package, or a mutant of its variable-length
module) and raises on a mismatch.

* The pages' two-key example ([CSW] "How can softmax be computed across tiles?") placed in a
  decoding step and in an over-full query chunk, with both causal alignments; the expected
  values are derived by hand in tests/golden/decode_two_key.json.
* Reductions to the square-attention oracle (itself pinned separately): equal lengths under
  either alignment; the last Lq rows of a causal prefill of Lk tokens (bottom-right alignment:
  chunked prefill); the first Lq keys under top-left alignment; a single decoding row seeing
  every key.
* Packing: a packed batch equals its sequences computed one at a time, and tokens outside every
  sequence stay untouched.
* A pure-Python brute force with exactly rounded sums on tiny packed inputs.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
CASES = [(False, "bottom_right"), (True, "bottom_right"), (True, "top_left")]


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f(x):
    return -math.inf if x == "-inf" else float(x)


def _rand(seed, T, H, d, scale=1.0):
    return np.random.default_rng(seed).standard_normal((T, H, d)) * scale


def _bhnd(x):
    """[T, H, d] (one sequence) -> [1, H, T, d]."""
    return np.ascontiguousarray(np.transpose(x, (1, 0, 2)))[None]


def _tok(x):
    """[1, H, T, d] -> [T, H, d]."""
    return np.transpose(x[0], (1, 0, 2))


def pin_varlen_decode_example(impl):
    g = _golden("decode_two_key.json")
    k = np.asarray(g["k"])[:, None, :]
    v = np.asarray(g["v"])[:, None, :]
    q1 = np.asarray(g["q_row"])[None, None, :]
    for key, causal, align in (("bottom_right", True, "bottom_right"), ("top_left", True, "top_left"),
                               ("no_mask", False, "bottom_right")):
        O, LSE = impl.attention_varlen_ref(q1, k, v, [0, 1], [0, 2], g["scale"], causal=causal, align=align)
        want = g["decode"][key]
        assert np.allclose(O[0, 0], want["O"], atol=1e-14), (key, O)
        assert abs(LSE[0, 0] - want["LSE"]) < 1e-14, (key, LSE)
    q3 = np.repeat(q1, 3, axis=0)
    O, LSE = impl.attention_varlen_ref(q3, k, v, [0, 3], [0, 2], g["scale"], causal=True, align="bottom_right")
    want = g["overfull_bottom_right"]
    for r in range(3):
        assert np.allclose(O[r, 0], want["O"][r], atol=1e-14), (r, O[r])
        wl = _f(want["LSE"][r])
        assert (LSE[0, r] == wl) if math.isinf(wl) else abs(LSE[0, r] - wl) < 1e-14, (r, LSE[0, r])


def pin_varlen_equal_lengths(impl):
    """Lq = Lk: both alignments are the square causal mask of the pinned square oracle."""
    q, k, v = (_rand(s, 23, 2, 5) for s in (1, 2, 3))
    for causal, align in CASES:
        O, LSE = impl.attention_varlen_ref(q, k, v, [0, 23], [0, 23], 0.6, causal=causal, align=align)
        Or, Lr = impl.attention_ref(_bhnd(q), _bhnd(k), _bhnd(v), 0.6, causal=causal)
        assert np.allclose(O, _tok(Or), atol=1e-13), (causal, align)
        assert np.allclose(LSE, Lr[0], atol=1e-13), (causal, align)


def pin_varlen_chunked_prefill(impl):
    """Bottom-right: the queries are the last Lq positions of the sequence, so they must equal
    rows Lk-Lq .. Lk-1 of a causal pass over all Lk tokens."""
    Lk, Lq = 29, 7
    q, k, v = (_rand(s, Lk, 2, 4) for s in (4, 5, 6))
    Of, Lf = impl.attention_ref(_bhnd(q), _bhnd(k), _bhnd(v), 0.7, causal=True)
    O, LSE = impl.attention_varlen_ref(q[Lk - Lq:], k, v, [0, Lq], [0, Lk], 0.7, causal=True, align="bottom_right")
    assert np.allclose(O, _tok(Of)[Lk - Lq:], atol=1e-13)
    assert np.allclose(LSE, Lf[0][:, Lk - Lq:], atol=1e-13)


def pin_varlen_top_left_prefix(impl):
    """Top-left with Lq <= Lk: row i sees keys 0..i, all inside the first Lq keys, so the result
    is the square causal pass over the first Lq tokens; with Lq > Lk rows i >= Lk see every key."""
    Lq, Lk = 9, 20
    q = _rand(7, Lq, 2, 4)
    k, v = _rand(8, Lk, 2, 4), _rand(9, Lk, 2, 4)
    O, LSE = impl.attention_varlen_ref(q, k, v, [0, Lq], [0, Lk], 0.5, causal=True, align="top_left")
    Or, Lr = impl.attention_ref(_bhnd(q), _bhnd(k[:Lq]), _bhnd(v[:Lq]), 0.5, causal=True)
    assert np.allclose(O, _tok(Or), atol=1e-13) and np.allclose(LSE, Lr[0], atol=1e-13)
    Lq2, Lk2 = 12, 5
    q2 = _rand(10, Lq2, 1, 3)
    k2, v2 = _rand(11, Lk2, 1, 3), _rand(12, Lk2, 1, 3)
    O2, L2 = impl.attention_varlen_ref(q2, k2, v2, [0, Lq2], [0, Lk2], 0.5, causal=True, align="top_left")
    On, Ln = impl.attention_ref(_bhnd(q2[Lk2:]), _bhnd(k2), _bhnd(v2), 0.5, causal=False)
    assert np.allclose(O2[Lk2:], _tok(On), atol=1e-13) and np.allclose(L2[:, Lk2:], Ln[0], atol=1e-13)


def pin_varlen_decode_sees_all(impl):
    """One query row under bottom-right alignment sees every key: the unmasked result; under
    top-left alignment it sees key 0 only: O = v_0, LSE = its score."""
    Lk = 37
    q = _rand(13, 1, 3, 8)
    k, v = _rand(14, Lk, 3, 8), _rand(15, Lk, 3, 8)
    Oc, Lc = impl.attention_varlen_ref(q, k, v, [0, 1], [0, Lk], 0.35, causal=True, align="bottom_right")
    On, Ln = impl.attention_varlen_ref(q, k, v, [0, 1], [0, Lk], 0.35, causal=False)
    Or, Lr = impl.attention_ref(_bhnd(q), _bhnd(k), _bhnd(v), 0.35)
    assert np.allclose(Oc, On, atol=1e-14) and np.allclose(Lc, Ln, atol=1e-14)
    assert np.allclose(On, _tok(Or), atol=1e-13) and np.allclose(Ln, Lr[0], atol=1e-13)
    Ot, Lt = impl.attention_varlen_ref(q, k, v, [0, 1], [0, Lk], 0.35, causal=True, align="top_left")
    assert np.allclose(Ot[0], v[0], atol=1e-14)
    assert np.allclose(Lt[:, 0], 0.35 * (q[0] * k[0]).sum(axis=1), atol=1e-14)


def pin_varlen_packing(impl):
    """A packed batch (lengths with an empty sequence and unequal query/key counts) equals its
    sequences computed one at a time; trailing tokens outside every sequence stay 0 / -inf."""
    lq = [5, 0, 3, 8]
    lk = [9, 4, 3, 2]
    cq = np.concatenate([[0], np.cumsum(lq)])
    ck = np.concatenate([[0], np.cumsum(lk)])
    Tq, Tk = int(cq[-1]) + 2, int(ck[-1]) + 1
    q = _rand(16, Tq, 3, 4)
    k, v = _rand(17, Tk, 3, 4), _rand(18, Tk, 3, 4)
    for causal, align in CASES:
        O, LSE = impl.attention_varlen_ref(q, k, v, cq, ck, 0.8, causal=causal, align=align)
        for b in range(len(lq)):
            qs, qe, ks, ke = cq[b], cq[b + 1], ck[b], ck[b + 1]
            O1, L1 = impl.attention_varlen_ref(q[qs:qe], k[ks:ke], v[ks:ke], [0, lq[b]], [0, lk[b]], 0.8,
                                               causal=causal, align=align)
            assert np.allclose(O[qs:qe], O1, atol=1e-14) and np.allclose(LSE[:, qs:qe], L1, atol=1e-14), (b, causal)
        assert not np.any(O[cq[-1]:]) and np.all(LSE[:, cq[-1]:] == -np.inf)


def pin_varlen_brute(impl):
    """Exactly rounded pure-Python loops on tiny packed inputs, every mask and alignment."""
    lq = [3, 1, 4, 2]
    lk = [2, 5, 4, 0]
    cq = [0] + list(np.cumsum(lq))
    ck = [0] + list(np.cumsum(lk))
    q = _rand(19, cq[-1], 2, 3, 1.5)
    k, v = _rand(20, ck[-1], 2, 3, 1.5), _rand(21, ck[-1], 2, 3)
    for causal, align in CASES:
        O, LSE = impl.attention_varlen_ref(q, k, v, cq, ck, 0.9, causal=causal, align=align)
        Ob, Lb = impl.brute_varlen_ref(q, k, v, cq, ck, 0.9, causal=causal, align=align)
        Ob, Lb = np.asarray(Ob), np.asarray(Lb)
        assert np.allclose(O, Ob, atol=1e-14, rtol=1e-13), (causal, align, np.abs(O - Ob).max())
        fin = np.isfinite(Lb)
        assert np.array_equal(fin, np.isfinite(LSE)) and np.allclose(LSE[fin], Lb[fin], atol=1e-13)


def pin_varlen_rejects_unknown_alignment(impl):
    q = _rand(22, 2, 1, 2)
    try:
        impl.attention_varlen_ref(q, q, q, [0, 2], [0, 2], 1.0, causal=True, align="diagonal")
    except ValueError:
        return
    raise AssertionError("an unknown causal alignment was accepted")


PINS = [pin_varlen_decode_example, pin_varlen_equal_lengths, pin_varlen_chunked_prefill, pin_varlen_top_left_prefix,
        pin_varlen_decode_sees_all, pin_varlen_packing, pin_varlen_brute, pin_varlen_rejects_unknown_alignment]
