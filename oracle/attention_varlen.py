"""fp64 CPU oracle for packed variable-length attention with unequal query and key lengths --
TEST INFRASTRUCTURE, not part of the product.

Only the test suite, the smoke check and the benchmark may import this module.  It shares no
code with the HIP path and imports nothing from it.

Sources (web pages, cited by title and section):

* [CSW] "FlashAttention Interview Questions: IO Complexity, Tiling, and Numerical
  Stability" (cswork.org).  Section "What is FlashAttention exact about?" fixes the target
  O = row_softmax(scale * Q K^T + mask) V for one head.  Section "Does subtracting the maximum
  solve every numerical issue?" warns that incremental decoding, unequal query and key lengths,
  padding and packed sequences each change which keys a query may see, and that this must be
  settled before numerical errors are compared.  Its closing benchmark section separates
  prefill (many query rows) from single-token decoding (one query row per sequence).

The pages name the cases but fix no convention for them, so the readings below are this
module's (also listed in the design notes):

* Packing.  Sequence b owns query tokens cu_q[b] .. cu_q[b+1]-1 and key/value tokens
  cu_k[b] .. cu_k[b+1]-1 of the packed tensors; Lq = cu_q[b+1] - cu_q[b], Lk likewise.
  Tensors are token-major: q and o are [Tq, H, d], k and v are [Tk, H, d]; the log-sum-exp is
  [H, Tq].  Sequences never see each other's keys.
* Causal alignment is explicit.  Query row i (0-based within its sequence) may see key j iff
  j <= i + delta, where delta = Lk - Lq under "bottom_right" alignment (the queries are the
  last Lq positions of a sequence whose keys are all Lk positions: decoding and chunked
  prefill) and delta = 0 under "top_left" alignment (query i and key i share a position).
  With Lq = Lk the two coincide.  Without the causal mask every key of the sequence is
  visible.
* A row with no visible key (bottom-right alignment with Lq > Lk, or Lk = 0) has output 0 and
  log-sum-exp -inf, as for the square case.

``attention_varlen_ref`` is the definition written out: for every sequence and head the whole
score matrix is materialised, the hidden entries are replaced by -inf, and each row is
normalised in two passes (maximum, then shifted exponentials and their sum).
"""

from __future__ import annotations

import math

import numpy as np

from .attention import _as_f64

ALIGNMENTS = ("bottom_right", "top_left")


def causal_offset(Lq: int, Lk: int, align: str) -> int:
    """delta of the reading above: query i may see key j iff j <= i + delta."""
    if align == "bottom_right":
        return Lk - Lq
    if align == "top_left":
        return 0
    raise ValueError(f"unknown causal alignment {align!r}; expected one of {ALIGNMENTS}")


def _lengths(cu, total):
    cu = [int(x) for x in (cu.tolist() if hasattr(cu, "tolist") else cu)]
    if cu[0] != 0 or any(b < a for a, b in zip(cu, cu[1:])) or cu[-1] > total:
        raise ValueError("cu_seqlens must start at 0, be non-decreasing and end within the tensor")
    return cu


def attention_varlen_ref(q, k, v, cu_seqlens_q, cu_seqlens_k, scale: float, causal: bool = False,
                         align: str = "bottom_right"):
    """Exact attention over packed sequences, in float64.

    Parameters
    ----------
    q : [Tq, H, d]; k, v : [Tk, H, d] (token-major, any float dtype, upcast exactly).
    cu_seqlens_q, cu_seqlens_k : int sequences [B + 1], prefix sums of the per-sequence query
        and key lengths (first entry 0).
    scale : multiplier of every dot product (the float32 value the kernel receives).
    causal : apply the causal mask with the given alignment.
    align : "bottom_right" or "top_left" (only used when causal).

    Returns
    -------
    (O, LSE): O [Tq, H, d] float64, LSE [H, Tq] float64 (natural log).  Query tokens that belong
    to no sequence (past cu_seqlens_q[-1]) are left at 0 / -inf.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    Tq, H, d = q.shape
    Tk = k.shape[0]
    cq = _lengths(cu_seqlens_q, Tq)
    ck = _lengths(cu_seqlens_k, Tk)
    if len(cq) != len(ck):
        raise ValueError("cu_seqlens_q and cu_seqlens_k describe different numbers of sequences")
    if causal:
        causal_offset(0, 0, align)          # reject an unknown alignment even for empty input
    c = float(scale)
    O = np.zeros((Tq, H, v.shape[2]), dtype=np.float64)
    LSE = np.full((H, Tq), -np.inf, dtype=np.float64)
    for b in range(len(cq) - 1):
        qs, qe, ks, ke = cq[b], cq[b + 1], ck[b], ck[b + 1]
        Lq, Lk = qe - qs, ke - ks
        if Lq == 0:
            continue
        # which keys each query row of this sequence may see
        i = np.arange(Lq)[:, None]
        j = np.arange(Lk)[None, :]
        ok = np.ones((Lq, Lk), dtype=bool)
        if causal:
            ok = j <= i + causal_offset(Lq, Lk, align)
        any_ok = ok.any(axis=1)
        for h in range(H):
            # full score matrix of this sequence and head, hidden entries selected to -inf
            s = np.where(ok, (q[qs:qe, h] @ k[ks:ke, h].T) * c, -np.inf)
            # first pass: row maximum over the visible keys
            m = np.where(any_ok, s.max(axis=1, initial=-np.inf), 0.0)
            # second pass: shifted exponentials, their sum, the normalised value sum
            p = np.where(ok, np.exp(s - m[:, None]), 0.0)
            l = p.sum(axis=1)
            o = (p @ v[ks:ke, h]) / np.where(any_ok, l, 1.0)[:, None]
            O[qs:qe, h] = np.where(any_ok[:, None], o, 0.0)
            LSE[h, qs:qe] = np.where(any_ok, m + np.log(np.where(any_ok, l, 1.0)), -np.inf)
    return O, LSE


def brute_varlen_ref(q, k, v, cu_seqlens_q, cu_seqlens_k, scale: float, causal: bool = False,
                     align: str = "bottom_right"):
    """Pure-Python loops with exactly rounded sums (``math.fsum``); tiny inputs only.

    Same arguments and reading as ``attention_varlen_ref``; nested lists or arrays in, nested
    lists out: O [Tq][H][d], LSE [H][Tq].
    """
    q = [[[float(x) for x in hv] for hv in t] for t in np.asarray(q, dtype=np.float64)]
    k = [[[float(x) for x in hv] for hv in t] for t in np.asarray(k, dtype=np.float64)]
    v = [[[float(x) for x in hv] for hv in t] for t in np.asarray(v, dtype=np.float64)]
    Tq, H, d = len(q), len(q[0]), len(v[0][0])
    cq = [int(x) for x in cu_seqlens_q]
    ck = [int(x) for x in cu_seqlens_k]
    O = [[[0.0] * d for _ in range(H)] for _ in range(Tq)]
    LSE = [[-math.inf] * Tq for _ in range(H)]
    for b in range(len(cq) - 1):
        Lq, Lk = cq[b + 1] - cq[b], ck[b + 1] - ck[b]
        for h in range(H):
            for i in range(Lq):
                tq = cq[b] + i
                vis = []
                for j in range(Lk):
                    if causal and align == "bottom_right" and j > i + (Lk - Lq):
                        continue
                    if causal and align == "top_left" and j > i:
                        continue
                    vis.append(ck[b] + j)
                if not vis:
                    continue
                s = {t: scale * math.fsum(q[tq][h][e] * k[t][h][e] for e in range(len(q[tq][h]))) for t in vis}
                mx = max(s.values())
                w = {t: math.exp(s[t] - mx) for t in vis}
                den = math.fsum(w.values())
                O[tq][h] = [math.fsum(w[t] * v[t][h][e] for t in vis) / den for e in range(d)]
                LSE[h][tq] = mx + math.log(den)
    return O, LSE
