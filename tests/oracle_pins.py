"""Pins that tie the fp64 oracle to what the pages and the mathematics fix.

Each pin takes an implementation namespace ``impl`` (the real ``oracle`` package, or a
mutated copy of it built by the mutation test) and raises ``AssertionError`` when the
implementation disagrees with a value printed on the pages, a closed form, an invariant,
a library routine or a brute-force evaluation.

Pages:
* [CSW] "FlashAttention Interview Questions: IO Complexity, Tiling, and Numerical
  Stability" (cswork.org).
* [LIQ] "FlashAttention 1, 2 & 3: Memory Tiling & Eliminating the O(N^2) HBM
  Bottleneck" (learn-interview-questions, Q18).
"""

from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import scipy.special

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _frac(x):
    return float(Fraction(*x)) if isinstance(x, list) else float(x)


def _h(x):
    """[N, d] -> [1, 1, N, d]."""
    return np.asarray(x, dtype=np.float64)[None, None]


def _two_tile_inputs(shift=0.0):
    """Query 0 reproduces the two-tile example: q0 = (1, shift), k_j = (s_j, 1), so the
    score of key j is s_j + shift.  Query 1 is an unrelated row."""
    g = _golden("two_tile_example.json")
    s = g["tile_scores"]
    vals = g["tile_values"]
    q = [[1.0, shift], [0.5, -0.25]]
    k = [[s[0], 1.0], [s[1], 1.0]]
    v = [[vals[0], -1.0], [vals[1], 3.0]]
    return np.array(q), np.array(k), np.array(v)


# --------------------------------------------------------------------------- pages' values

def pin_two_tile_output(impl):
    """[CSW] "How can softmax be computed across tiles?": the example's output is 5."""
    g = _golden("two_tile_example.json")
    q, k, v = _two_tile_inputs()
    O, LSE = impl.attention_ref(_h(q), _h(k), _h(v), 1.0)
    assert abs(O[0, 0, 0, 0] - g["output"]) < 1e-13, O[0, 0, 0, 0]
    # full-softmax weights 1/4 and 3/4 give l = 1 + 3 in the frame of the first score
    assert abs(LSE[0, 0, 0] - math.log(4.0)) < 1e-13
    assert abs(g["normalise_each_tile_then_average"] - g["output"]) > 0.5


def pin_two_tile_weights(impl):
    """[CSW] same example: a full softmax gives weights 1/4 and 3/4."""
    g = _golden("two_tile_example.json")
    q, k, _ = _two_tile_inputs()
    w = impl.softmax_weights_ref(q, k, 1.0)
    want = [_frac(x) for x in g["full_softmax_weights"]]
    assert np.allclose(w[0], want, rtol=0, atol=1e-15), w[0]


def pin_two_tile_intermediates(impl):
    """[CSW] same example through the running update with singleton tiles:
    m=0, l=1, a=2 after tile 1; l=4/3, a=20/3 after tile 2; output 5."""
    g = _golden("two_tile_example.json")
    q, k, v = _two_tile_inputs()
    O, LSE, hist = impl.online_ref(q, k, v, 1.0, tiles=[1, 1])
    (m1, l1, a1), (m2, l2, a2) = hist[0]
    t1, t2 = g["after_tile_1"], g["after_tile_2"]
    assert abs(m1 - t1["m"]) < 1e-15 and abs(l1 - t1["l"]) < 1e-15 and abs(a1[0] - t1["a"]) < 1e-15
    assert abs(m2 - t2["m"]) < 1e-15
    assert abs(l2 - _frac(t2["l"])) < 1e-14, l2
    assert abs(a2[0] - _frac(t2["a"])) < 1e-14, a2
    assert abs(O[0, 0] - g["output"]) < 1e-14
    # the rescale factor applied to the first tile's statistics is exp(m1 - m2) = 1/3
    assert abs(math.exp(m1 - m2) - _frac(g["rescale_factor"])) < 1e-15


def pin_two_tile_brute(impl):
    """[CSW] same example through the brute-force evaluator."""
    g = _golden("two_tile_example.json")
    q, k, v = _two_tile_inputs()
    O, LSE = impl.brute_ref(q, k, v, 1.0)
    assert abs(O[0][0] - g["output"]) < 1e-14
    assert abs(LSE[0] - math.log(4.0)) < 1e-14


def pin_shift_1000(impl):
    """[CSW] "Does subtracting the maximum solve every numerical issue?": adding 1,000 to
    both scores still returns about 5; raw exponentials overflow in float64."""
    g = _golden("shift_example.json")
    q, k, v = _two_tile_inputs(shift=g["shift"])
    with np.errstate(over="ignore"):
        assert not np.isfinite(np.exp(np.array(g["tile_scores"]) + g["shift"])).all()
    O, LSE = impl.attention_ref(_h(q), _h(k), _h(v), 1.0)
    assert abs(O[0, 0, 0, 0] - g["output"]) < 1e-12, O[0, 0, 0, 0]
    assert abs(LSE[0, 0, 0] - (g["shift"] + math.log(4.0))) < 1e-12
    O2, LSE2, _ = impl.online_ref(q, k, v, 1.0, tiles=[1, 1])
    assert abs(O2[0, 0] - g["output"]) < 1e-12
    O3, LSE3 = impl.brute_ref(q, k, v, 1.0)
    assert abs(O3[0][0] - g["output"]) < 1e-12


def pin_large_spread(impl):
    """[CSW] same section: subtracting the *maximum* keeps every shifted exponential <= 1.
    Scores 0 and 1000: the output is the value of the larger score (to e^-1000) and the
    LSE is 1000 (+ e^-1000); shifting by anything smaller than the maximum overflows."""
    q = np.array([[1.0, 1000.0]])
    k = np.array([[0.0, 0.0], [0.0, 1.0]])
    v = np.array([[-7.0, 1.0], [2.0, 3.0]])
    O, LSE = impl.attention_ref(_h(q), _h(k), _h(v), 1.0)
    assert np.array_equal(O[0, 0, 0], v[1]), O[0, 0, 0]
    assert LSE[0, 0, 0] == 1000.0
    O2, LSE2, _ = impl.online_ref(q, k, v, 1.0, tiles=[1, 1])
    assert np.array_equal(O2[0], v[1]) and LSE2[0] == 1000.0
    O2, LSE2, _ = impl.online_ref(q, k, v, 1.0, tiles=[2])
    assert np.array_equal(O2[0], v[1]) and LSE2[0] == 1000.0
    # the large score first: the running maximum must keep it when a smaller tile follows
    O3, LSE3, _ = impl.online_ref(q, k[::-1], v[::-1], 1.0, tiles=[1, 1])
    assert np.array_equal(O3[0], v[1]) and LSE3[0] == 1000.0


def pin_memory_budget(impl):
    """[CSW] "Which complexity becomes smaller, and which does not?": payload table."""
    g = _golden("memory_budget.json")
    a = impl.accounting
    N, d, e = g["N"], g["d"], g["bytes_per_element"]
    MiB = 1 << 20
    assert a.score_matrix_elements(N) == g["score_matrix_elements"]
    assert a.score_matrix_bytes(N, e) == g["score_matrix_MiB"] * MiB
    assert a.head_tensor_elements(N, d) == g["head_tensor_elements"]
    assert a.head_tensor_bytes(N, d, e) == g["head_tensor_MiB"] * MiB
    assert a.qkvo_bytes(N, d, e) == g["qkvo_MiB"] * MiB
    dn = g["doubled_N"]
    assert a.score_matrix_bytes(dn["N"], e) == dn["score_matrix_MiB"] * MiB
    assert a.head_tensor_bytes(dn["N"], d, e) == dn["head_tensor_MiB"] * MiB


def pin_element_counts(impl):
    """[LIQ] section 1: 8,000 tokens -> 64,000,000 scores; 64,000 -> 4,096,000,000."""
    g = _golden("element_counts.json")
    for c in g["cases"]:
        assert impl.accounting.score_matrix_elements(c["N"]) == c["score_matrix_elements"]


# --------------------------------------------------------------------------- closed forms

def _geom(beta, n):
    """Closed forms for scores beta*j, values j, j = 0..n-1:
    returns (sum_j j r^j / sum_j r^j, ln sum_j r^j) with r = e^beta (beta != 0)."""
    r = math.exp(beta)
    S0 = (1 - r ** n) / (1 - r)
    S1 = r * (1 - n * r ** (n - 1) + (n - 1) * r ** n) / (1 - r) ** 2
    return S1 / S0, math.log(S0)


def pin_geometric_closed_form(impl):
    """d = 1, q_i = 1, k_j = beta*j, v_j = j: the weights are geometric, so the output and
    LSE have closed forms.  Checked non-causal (n = N keys), causal (n = i+1 keys for row
    i) and with key padding (n = L).  Catches off-by-one masks, transposed operands and
    wrong value rows, since every key carries a distinct value."""
    N, beta = 9, 0.3
    q = np.ones((N, 1))
    k = beta * np.arange(N, dtype=np.float64)[:, None]
    v = np.arange(N, dtype=np.float64)[:, None]
    O, LSE = impl.attention_ref(_h(q), _h(k), _h(v), 1.0)
    want_o, want_l = _geom(beta, N)
    assert np.allclose(O[0, 0, :, 0], want_o, rtol=0, atol=1e-12)
    assert np.allclose(LSE[0, 0], want_l, rtol=0, atol=1e-12)
    O, LSE = impl.attention_ref(_h(q), _h(k), _h(v), 1.0, causal=True)
    for i in range(N):
        if i == 0:
            wo, wl = 0.0, 0.0
        else:
            wo, wl = _geom(beta, i + 1)
        assert abs(O[0, 0, i, 0] - wo) < 1e-12, (i, O[0, 0, i, 0], wo)
        assert abs(LSE[0, 0, i] - wl) < 1e-12
    L = 5
    O, LSE = impl.attention_ref(_h(q), _h(k), _h(v), 1.0, seqlens=[L])
    wo, wl = _geom(beta, L)
    assert np.allclose(O[0, 0, :, 0], wo, rtol=0, atol=1e-12)
    assert np.allclose(LSE[0, 0], wl, rtol=0, atol=1e-12)
    # the same through the running update and the brute-force evaluator
    O2, LSE2, _ = impl.online_ref(q, k, v, 1.0, tiles=[2, 3, 4], causal=True)
    Ob, LSEb = impl.brute_ref(q, k, v, 1.0, causal=True)
    for i in range(1, N):
        wo, wl = _geom(beta, i + 1)
        assert abs(O2[i, 0] - wo) < 1e-12 and abs(LSE2[i] - wl) < 1e-12
        assert abs(Ob[i][0] - wo) < 1e-12 and abs(LSEb[i] - wl) < 1e-12


def pin_q_zero_mean(impl):
    """Q = 0 makes every visible score 0: the output is the mean of the visible value
    rows and the LSE is ln(count).  Non-causal: mean of all rows; causal: prefix means;
    key padding: mean of the first L rows."""
    rng = np.random.default_rng(11)
    N, d = 13, 6
    q = np.zeros((N, d))
    k = rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    O, LSE = impl.attention_ref(_h(q), _h(k), _h(v), 0.37)
    assert np.allclose(O[0, 0], v.mean(axis=0)[None], rtol=0, atol=1e-14)
    assert np.allclose(LSE[0, 0], math.log(N), rtol=0, atol=1e-14)
    O, LSE = impl.attention_ref(_h(q), _h(k), _h(v), 0.37, causal=True)
    prefix = np.cumsum(v, axis=0) / np.arange(1, N + 1)[:, None]
    assert np.allclose(O[0, 0], prefix, rtol=0, atol=1e-14)
    assert np.allclose(LSE[0, 0], np.log(np.arange(1, N + 1)), rtol=0, atol=1e-14)
    L = 4
    O, LSE = impl.attention_ref(_h(q), _h(k), _h(v), 0.37, seqlens=[L])
    assert np.allclose(O[0, 0], v[:L].mean(axis=0)[None], rtol=0, atol=1e-14)
    assert np.allclose(LSE[0, 0], math.log(L), rtol=0, atol=1e-14)
    O, LSE = impl.attention_ref(_h(q), _h(k), _h(v), 0.37, causal=True, seqlens=[L])
    both = np.cumsum(v[:L], axis=0) / np.arange(1, L + 1)[:, None]
    assert np.allclose(O[0, 0, :L], both, rtol=0, atol=1e-14)
    assert np.allclose(O[0, 0, L:], both[-1][None], rtol=0, atol=1e-14)


def pin_dominant_logit(impl):
    """One dominant logit selects its value row: keys one-hot (k_j = e_j), query i equal
    to (40/scale) e_{t(i)} gives score 40 on key t(i) and 0 elsewhere, so
    O_i = v_{t(i)} up to N e^-40 max|v| and LSE_i = 40 + ln(1 + (N-1) e^-40)."""
    rng = np.random.default_rng(5)
    N = d = 8
    scale = 0.125
    k = np.eye(N)
    v = rng.standard_normal((N, d))
    target = rng.permutation(N)
    q = np.zeros((N, d))
    q[np.arange(N), target] = 40.0 / scale
    O, LSE = impl.attention_ref(_h(q), _h(k), _h(v), scale)
    tol = N * math.exp(-40.0) * np.abs(v).max() * 2
    assert np.abs(O[0, 0] - v[target]).max() < tol
    assert np.allclose(LSE[0, 0], 40.0 + math.log1p((N - 1) * math.exp(-40.0)), rtol=0, atol=1e-13)


def pin_rows_sum_to_one(impl):
    """With V = identity (d = number of keys) the output row equals the softmax weights:
    each row sums to 1, hidden keys weigh exactly 0, and the weights match the
    library routine scipy.special.softmax over the visible scores."""
    rng = np.random.default_rng(7)
    N, dq = 11, 5
    q = rng.standard_normal((N, dq)) * 2
    k = rng.standard_normal((N, dq)) * 2
    v = np.eye(N)
    for causal, L in [(False, None), (True, None), (False, 7), (True, 7)]:
        O, LSE = impl.attention_ref(_h(q), _h(k), _h(v), 0.6, causal=causal,
                                    seqlens=None if L is None else [L])
        W = O[0, 0]
        assert np.allclose(W.sum(axis=1), 1.0, rtol=0, atol=1e-14)
        LL = N if L is None else L
        S = (q @ k.T) * 0.6
        for i in range(N):
            vis = [j for j in range(N) if j < LL and (not causal or j <= i)]
            hid = [j for j in range(N) if j not in vis]
            assert np.all(W[i, hid] == 0.0)
            assert np.allclose(W[i, vis], scipy.special.softmax(S[i, vis]), rtol=0, atol=1e-14)
            assert abs(LSE[0, 0, i] - scipy.special.logsumexp(S[i, vis])) < 1e-13
        Wr = impl.softmax_weights_ref(q, k, 0.6, causal=causal, seqlen=L)
        assert np.allclose(Wr, W, rtol=0, atol=1e-15)


# --------------------------------------------------------------------------- invariants

def pin_permutation(impl):
    """Non-causal, no padding: permuting the key and value rows together leaves every
    output unchanged; permuting query rows permutes the outputs."""
    rng = np.random.default_rng(3)
    N, d = 17, 8
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    O, LSE = impl.attention_ref(_h(q), _h(k), _h(v), 0.4)
    p = rng.permutation(N)
    O2, LSE2 = impl.attention_ref(_h(q), _h(k[p]), _h(v[p]), 0.4)
    assert np.allclose(O, O2, rtol=0, atol=1e-13) and np.allclose(LSE, LSE2, rtol=0, atol=1e-13)
    O3, LSE3 = impl.attention_ref(_h(q[p]), _h(k), _h(v), 0.4)
    assert np.allclose(O3[0, 0], O[0, 0, p], rtol=0, atol=1e-13)
    # and permuting the keys alone (values fixed) does change the result
    O4, _ = impl.attention_ref(_h(q), _h(k[p]), _h(v), 0.4)
    assert not np.allclose(O4, O, rtol=0, atol=1e-6)


def pin_tiling_invariance(impl):
    """[CSW] "Does subtracting the maximum ...": one full tile, singleton tiles, uneven
    partitions, and a late tile whose maximum is far larger than the earlier ones all
    agree with the two-pass reference, for every mask kind."""
    rng = np.random.default_rng(23)
    N, d = 19, 4
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    k_late = k.copy()
    k_late[-3:] *= 25.0          # the last tile raises the maximum by a lot
    parts = [[N], [1] * N, [1, 3, 2, 7, 6], [5, 5, 5, 4], [18, 1]]
    for kk in (k, k_late):
        for causal, L in [(False, None), (True, None), (False, 12), (True, 12)]:
            O, LSE = impl.attention_ref(_h(q), _h(kk), _h(v), 0.5, causal=causal,
                                        seqlens=None if L is None else [L])
            for tiles in parts:
                O2, LSE2, _ = impl.online_ref(q, kk, v, 0.5, tiles=tiles, causal=causal, seqlen=L)
                assert np.allclose(O2, O[0, 0], rtol=1e-12, atol=1e-12), (tiles, causal, L)
                assert np.allclose(LSE2, LSE[0, 0], rtol=1e-12, atol=1e-12)


def pin_masked_extremes(impl):
    """[CSW] same section: extreme numbers in masked positions leave every eligible
    output unchanged.  Padding: rows >= L of K and V set to +-3e38 (finite in bf16);
    causal: rows >= j0 of K and V set to extremes leave query rows < j0 unchanged."""
    rng = np.random.default_rng(29)
    N, d, L = 12, 4, 7
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    O, LSE = impl.attention_ref(_h(q), _h(k), _h(v), 0.5, seqlens=[L])
    k2, v2 = k.copy(), v.copy()
    k2[L:] = 3.0e38 * np.sign(rng.standard_normal((N - L, d)))
    v2[L:] = -3.0e38
    O2, LSE2 = impl.attention_ref(_h(q), _h(k2), _h(v2), 0.5, seqlens=[L])
    assert np.array_equal(O, O2) and np.array_equal(LSE, LSE2)
    j0 = 5
    Oc, LSEc = impl.attention_ref(_h(q), _h(k), _h(v), 0.5, causal=True)
    k3, v3 = k.copy(), v.copy()
    k3[j0:] = 1.0e4
    v3[j0:] = -3.0e38
    Oc2, LSEc2 = impl.attention_ref(_h(q), _h(k3), _h(v3), 0.5, causal=True)
    assert np.array_equal(Oc[0, 0, :j0], Oc2[0, 0, :j0])
    assert np.array_equal(LSEc[0, 0, :j0], LSEc2[0, 0, :j0])
    O4, _, _ = impl.online_ref(q, k2, v2, 0.5, tiles=[3, 4, 5], seqlen=L)
    assert np.allclose(O4, O[0, 0], rtol=1e-12, atol=1e-12)


def pin_special_cases(impl):
    """Textbook reductions: N = 1 gives O = v_0 and LSE = s_00; causal row 0 gives
    O_0 = v_0; L = 1 gives v_0 for every row; L = 0 gives O = 0 and LSE = -inf (the
    all-masked-row convention) with no NaN."""
    rng = np.random.default_rng(31)
    d = 6
    q, k, v = (rng.standard_normal((1, d)) for _ in range(3))
    O, LSE = impl.attention_ref(_h(q), _h(k), _h(v), 0.7)
    assert np.array_equal(O[0, 0, 0], v[0])
    assert abs(LSE[0, 0, 0] - 0.7 * float(q[0] @ k[0])) < 1e-14
    N = 9
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    O, LSE = impl.attention_ref(_h(q), _h(k), _h(v), 0.7, causal=True)
    assert np.array_equal(O[0, 0, 0], v[0])
    O, LSE = impl.attention_ref(_h(q), _h(k), _h(v), 0.7, seqlens=[1])
    assert np.array_equal(O[0, 0], np.repeat(v[:1], N, axis=0))
    for causal in (False, True):
        O, LSE = impl.attention_ref(_h(q), _h(k), _h(v), 0.7, causal=causal, seqlens=[0])
        assert np.array_equal(O, np.zeros_like(O)) and np.all(LSE == -np.inf)
        O2, LSE2, _ = impl.online_ref(q, k, v, 0.7, tiles=[4, 5], causal=causal, seqlen=0)
        assert np.array_equal(O2, np.zeros_like(O2)) and np.all(LSE2 == -np.inf)
        O3, LSE3 = impl.brute_ref(q, k, v, 0.7, causal=causal, seqlen=0)
        assert all(x == 0.0 for row in O3 for x in row) and all(x == -math.inf for x in LSE3)


def pin_brute_force(impl):
    """Brute force (pure Python, exactly rounded sums) on tiny inputs for every mask
    kind agrees with the matrix form and with the running update to 1e-13."""
    rng = np.random.default_rng(37)
    for N, d in [(1, 1), (2, 3), (5, 4), (8, 2)]:
        q, k, v = (rng.standard_normal((N, d)) * 1.5 for _ in range(3))
        for causal in (False, True):
            for L in (None, 1, max(1, N - 1), N):
                O, LSE = impl.attention_ref(_h(q), _h(k), _h(v), 0.8, causal=causal,
                                            seqlens=None if L is None else [L])
                Ob, LSEb = impl.brute_ref(q, k, v, 0.8, causal=causal, seqlen=L)
                assert np.allclose(O[0, 0], np.array(Ob), rtol=0, atol=1e-13), (N, d, causal, L)
                assert np.allclose(LSE[0, 0], np.array(LSEb), rtol=0, atol=1e-13)


def pin_batched_heads_independent(impl):
    """[CSW] "Batch size and head count multiply": each (b, h) is an independent head,
    and per-batch key lengths apply to their own batch element; sampled rows equal the
    corresponding rows of the full result."""
    rng = np.random.default_rng(41)
    B, H, N, d = 2, 3, 10, 4
    q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    seq = [6, 10]
    O, LSE = impl.attention_ref(q, k, v, 0.5, causal=True, seqlens=seq)
    for b in range(B):
        for h in range(H):
            Ob, LSEb = impl.brute_ref(q[b, h], k[b, h], v[b, h], 0.5, causal=True, seqlen=seq[b])
            assert np.allclose(O[b, h], np.array(Ob), rtol=0, atol=1e-13)
            assert np.allclose(LSE[b, h], np.array(LSEb), rtol=0, atol=1e-13)
    rows = np.array([[[0, 3, 9], [1, 2, 8], [4, 5, 6]], [[9, 7, 0], [3, 3, 3], [0, 1, 2]]])
    Os, LSEs = impl.attention_ref(q, k, v, 0.5, causal=True, seqlens=seq, rows=rows)
    for b in range(B):
        for h in range(H):
            assert np.array_equal(Os[b, h], O[b, h, rows[b, h]])
            assert np.array_equal(LSEs[b, h], LSE[b, h, rows[b, h]])


PINS = [
    pin_two_tile_output,
    pin_two_tile_weights,
    pin_two_tile_intermediates,
    pin_two_tile_brute,
    pin_shift_1000,
    pin_large_spread,
    pin_memory_budget,
    pin_element_counts,
    pin_geometric_closed_form,
    pin_q_zero_mean,
    pin_dominant_logit,
    pin_rows_sum_to_one,
    pin_permutation,
    pin_tiling_invariance,
    pin_masked_extremes,
    pin_special_cases,
    pin_brute_force,
    pin_batched_heads_independent,
]
