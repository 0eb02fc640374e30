"""Pins of the fp64 attention-gradient oracle: what the pages and the mathematics fix.

Each pin takes an ``impl`` (the oracle package, or a mutant of it) and raises on a mismatch.

* The pages' two-tile example, differentiated by hand ([CSW] "How can softmax be computed
  across tiles?", tests/golden/two_tile_grad.json).
* Central finite differences of the *forward* oracle, on tiny inputs, for every mask kind:
  the gradient is pinned to the forward definition, not to its own formula.
* Exact invariants of the gradient of a row softmax followed by P V: value-gradient columns
  sum to the upstream gradient, translating every key by one vector changes nothing, hidden
  keys receive nothing, the gradient is linear in the upstream gradient, and the softmax row
  term equals dO . O.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
MASKS = [(False, None), (True, None), (False, [3]), (True, [4])]


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _frac(x):
    return x[0] / x[1]


def _h(x):
    return np.asarray(x, dtype=np.float64)[None, None]


def _rand(seed, N=5, d=3, Nk=None):
    g = np.random.default_rng(seed)
    Nk = N if Nk is None else Nk
    return (g.standard_normal((1, 1, N, d)), g.standard_normal((1, 1, Nk, d)),
            g.standard_normal((1, 1, Nk, d)), g.standard_normal((1, 1, N, d)))


def pin_bwd_two_tile(impl):
    """[CSW] two-tile example with dO0 = (1, 0): dV, dQ and dK as derived by hand."""
    g = _golden("two_tile_grad.json")
    dq, dk, dv = impl.attention_bwd_ref(_h(g["q"]), _h(g["k"]), _h(g["v"]), _h(g["do"]), g["scale"])
    want_dv = np.array([[_frac(x) for x in row] for row in g["dV"]])
    want_dk = np.array([[_frac(x) for x in row] for row in g["dK"]])
    assert np.allclose(dv[0, 0], want_dv, atol=1e-14), dv
    assert np.allclose(dk[0, 0], want_dk, atol=1e-14), dk
    assert abs(dq[0, 0, 0, 0] - _frac(g["dQ0_first_component_over_ln3"]) * math.log(3.0)) < 1e-14, dq
    assert abs(dq[0, 0, 0, 1]) < 1e-14
    o, _ = impl.attention_ref(_h(g["q"]), _h(g["k"]), _h(g["v"]), g["scale"])
    assert abs(float(impl.row_dot_ref(o, _h(g["do"]))[0, 0, 0]) - g["row_term_D"]) < 1e-13


def pin_bwd_finite_differences(impl):
    """Central differences of L = sum(O * G) through the forward oracle, every mask kind."""
    h = 1e-5
    for mi, (causal, seq) in enumerate(MASKS):
        q, k, v, G = _rand(100 + mi)
        dq, dk, dv = impl.attention_bwd_ref(q, k, v, G, 0.7, causal=causal, seqlens=seq)

        def loss(q_, k_, v_):
            o, _ = impl.attention_ref(q_, k_, v_, 0.7, causal=causal, seqlens=seq)
            return float((o * G).sum())

        for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp = x.copy()
                xm = x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = {"q": q, "k": k, "v": v}
                args_m = {"q": q, "k": k, "v": v}
                args_p[name] = xp
                args_m[name] = xm
                num[idx] = (loss(**{a + "_": b for a, b in args_p.items()}) -
                            loss(**{a + "_": b for a, b in args_m.items()})) / (2 * h)
            err = np.abs(num - grad).max()
            assert err < 1e-7, (name, causal, seq, err)


def pin_bwd_value_columns(impl):
    """Rows of P sum to one, so sum_j dV_j = sum of dO over rows that see any key."""
    for mi, (causal, seq) in enumerate(MASKS):
        q, k, v, G = _rand(200 + mi, N=7, d=4)
        _, _, dv = impl.attention_bwd_ref(q, k, v, G, 0.5, causal=causal, seqlens=seq)
        L = 7 if seq is None else seq[0]
        sees = np.array([L > 0 for _ in range(7)])
        assert np.allclose(dv[0, 0].sum(axis=0), G[0, 0][sees].sum(axis=0), atol=1e-12)


def pin_bwd_key_translation(impl):
    """Adding one vector u to every key adds the constant scale*q_i.u to row i's scores: the
    softmax, the output and every gradient are unchanged."""
    for mi, (causal, seq) in enumerate(MASKS):
        q, k, v, G = _rand(300 + mi, N=6, d=3)
        u = np.array([0.3, -1.1, 0.6])
        a = impl.attention_bwd_ref(q, k, v, G, 0.8, causal=causal, seqlens=seq)
        b = impl.attention_bwd_ref(q, k + u, v, G, 0.8, causal=causal, seqlens=seq)
        for x, y in zip(a, b):
            assert np.allclose(x, y, atol=1e-12), np.abs(x - y).max()


def pin_bwd_hidden_keys(impl):
    """A key no row may see gets zero gradient; so does every key past the valid length."""
    q, k, v, G = _rand(400, N=6, d=3)
    _, dk, dv = impl.attention_bwd_ref(q, k, v, G, 0.9, seqlens=[4])
    assert np.all(dk[0, 0, 4:] == 0) and np.all(dv[0, 0, 4:] == 0)
    assert np.abs(dk[0, 0, :4]).max() > 0 and np.abs(dv[0, 0, :4]).max() > 0
    # causal: the last key is seen only by the last row, whose gradient decides it alone
    G2 = G.copy()
    G2[0, 0, -1] = 0.0
    _, dk2, dv2 = impl.attention_bwd_ref(q, k, v, G2, 0.9, causal=True)
    assert np.all(dv2[0, 0, -1] == 0) and np.all(dk2[0, 0, -1] == 0)
    # a row with no visible key (valid length 0) contributes nothing anywhere
    dq0, dk0, dv0 = impl.attention_bwd_ref(q, k, v, G, 0.9, seqlens=[0])
    assert not np.any(dq0) and not np.any(dk0) and not np.any(dv0)


def pin_bwd_linear_in_upstream(impl):
    """The gradient is linear in dO."""
    q, k, v, G = _rand(500, N=5, d=4)
    G2 = np.random.default_rng(501).standard_normal(G.shape)
    a = impl.attention_bwd_ref(q, k, v, G, 0.6, causal=True)
    b = impl.attention_bwd_ref(q, k, v, G2, 0.6, causal=True)
    c = impl.attention_bwd_ref(q, k, v, 2.0 * G - 3.0 * G2, 0.6, causal=True)
    for x, y, z in zip(a, b, c):
        assert np.allclose(2.0 * x - 3.0 * y, z, atol=1e-12)


def pin_bwd_batched_heads(impl):
    """Each (batch, head) is an independent attention: a batched call equals per-head calls."""
    g = np.random.default_rng(600)
    q, k, v, G = (g.standard_normal((2, 3, 5, 4)) for _ in range(4))
    seq = [5, 2]
    full = impl.attention_bwd_ref(q, k, v, G, 0.5, causal=True, seqlens=seq)
    for b in range(2):
        for hh in range(3):
            one = impl.attention_bwd_ref(q[b:b + 1, hh:hh + 1], k[b:b + 1, hh:hh + 1], v[b:b + 1, hh:hh + 1],
                                         G[b:b + 1, hh:hh + 1], 0.5, causal=True, seqlens=[seq[b]])
            for x, y in zip(full, one):
                assert np.allclose(x[b, hh], y[0, 0], atol=1e-14)


def pin_bwd_row_term(impl):
    """The softmax row term D_i = sum_j P_ij dP_ij equals dO_i . O_i (identity), here with the
    forward oracle's weights and output on random data."""
    q, k, v, G = _rand(700, N=6, d=4)
    o, _ = impl.attention_ref(q, k, v, 0.8, causal=True)
    w = impl.softmax_weights_ref(q[0, 0], k[0, 0], 0.8, causal=True)
    d_alt = (w * (G[0, 0] @ v[0, 0].T)).sum(axis=1)
    assert np.allclose(impl.row_dot_ref(o, G)[0, 0], d_alt, atol=1e-13)


PINS = [pin_bwd_two_tile, pin_bwd_row_term, pin_bwd_finite_differences, pin_bwd_value_columns, pin_bwd_key_translation,
        pin_bwd_hidden_keys, pin_bwd_linear_in_upstream, pin_bwd_batched_heads]
