"""fp64 CPU oracle for exact attention -- TEST INFRASTRUCTURE, not part of the product.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import
this module.  It shares no code with the HIP path and imports nothing from it.

Sources (web pages, cited by title and section):

* [CSW] "FlashAttention Interview Questions: IO Complexity, Tiling, and Numerical
  Stability" (cswork.org).  Section "What is FlashAttention exact about?" gives the
  target: scores = Q K^T / sqrt(d); weights = row_softmax(scores + mask);
  output = weights V, for one head of length N and width d.  Section "How can
  softmax be computed across tiles?" gives the running-statistics update (running
  maximum m, shifted sum l, unnormalised accumulator a, rescaled by exp(m - m_new)
  when a tile raises the maximum) and a two-tile worked example.  Section "Does
  subtracting the maximum solve every numerical issue?" gives the shift-invariance
  exercise and requires masked tiles to add no probability mass and an explicit
  convention for rows whose every key is masked.
* [LIQ] "FlashAttention 1, 2 & 3: Memory Tiling & Eliminating the O(N^2) HBM
  Bottleneck" (learn-interview-questions, Q18), section 1: the same softmax(QK^T/sqrt(d))V.

Because the tiled method reaches exactly the plain definition (up to rounding
order), ``attention_ref`` is that definition written out in float64: each query
row's full score row is materialised, a first pass finds the row maximum and a
second pass exponentiates, sums and normalises.  No tiling, no online update.

Readings of points the pages leave open (each also listed in the design notes):

* Layout: tensors are [B, H, N, d]; a batch-and-head pair is one independent head.
* ``scale`` multiplies the raw dot products (the pages' 1/sqrt(d)); callers pass
  the float32 value the kernel receives.
* The mask is applied by *selecting* -inf (weight exactly 0) for keys a query may
  not see, never by adding a large negative number.  Key j is visible to query i
  iff j < L (L = clamp(seqlens[b], 0, N) under key padding, else N) and, under the
  causal mask, j <= i (square, aligned query and key positions).
* Key padding masks keys only; query rows at or beyond L are computed normally.
* A row with no visible key has output 0 and log-sum-exp -inf (never NaN).
* LSE is the natural-log log-sum-exp of the visible scaled scores, m + ln l.
"""

from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np


def _as_f64(x) -> np.ndarray:
    """Exact upcast to float64 (bf16/fp16/fp32 values are representable exactly)."""
    if hasattr(x, "detach"):  # a torch tensor: go through float32, which holds bf16 exactly
        x = x.detach().cpu().float().numpy()
    return np.asarray(x, dtype=np.float64)


def visible_keys(i: np.ndarray, L: int, causal: bool, n_keys: int) -> np.ndarray:
    """Boolean [len(i), n_keys]: may query row i see key j?  (causal: j <= i; padding: j < L)."""
    j = np.arange(n_keys)[None, :]
    ok = j < L
    if causal:
        ok = ok & (j <= np.asarray(i)[:, None])
    return ok


def attention_ref(q, k, v, scale: float, causal: bool = False, seqlens=None,
                  rows=None, row_block: int = 256):
    """Exact attention in float64, one score row block at a time.

    Parameters
    ----------
    q : array-like [B, H, N, d]; k, v : [B, H, Nk, d] (Nk = N for self-attention);
        any float dtype, upcast to float64.
    scale : multiplier applied to every dot product q_i . k_j.
    causal : hide keys j > i.
    seqlens : optional int sequence [B]; keys j >= seqlens[b] are hidden.
    rows : optional query rows to compute: int array [R] (same for every head) or
        [B, H, R].  Default: all N rows.

    Returns
    -------
    (O, LSE): O [B, H, R, d] float64, LSE [B, H, R] float64 (natural log).
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    B, H, N, d = q.shape
    Nk = k.shape[2]                     # number of keys (equal to N for self-attention)
    dv = v.shape[3]                     # value width (equal to d in the kernel's contract)
    if rows is None:
        R = N
    else:
        rows = np.asarray(rows if not hasattr(rows, "numpy") else rows.cpu().numpy(), dtype=np.int64)
        R = rows.shape[-1]
    O = np.zeros((B, H, R, dv), dtype=np.float64)
    LSE = np.full((B, H, R), -np.inf, dtype=np.float64)
    c = float(scale)
    for b in range(B):
        L = Nk
        if seqlens is not None:
            L = int(min(max(int(seqlens[b]), 0), Nk))
        for h in range(H):
            if rows is None:
                idx_all = np.arange(N)
            elif rows.ndim == 1:
                idx_all = rows
            else:
                idx_all = rows[b, h]
            Kb = k[b, h, :L]            # keys a query could ever see
            Vb = v[b, h, :L]
            for r0 in range(0, R, row_block):
                idx = idx_all[r0:r0 + row_block]
                # step 1: full score rows s_ij = c * q_i . k_j
                s = (q[b, h, idx] @ Kb.T) * c
                # step 2: select -inf where the mask hides the key
                ok = visible_keys(idx, L, causal, L)
                s = np.where(ok, s, -np.inf)
                any_ok = ok.any(axis=1)
                # step 3: first pass, row maximum over visible keys
                m = np.where(any_ok, s.max(axis=1, initial=-np.inf), 0.0)
                # step 4: second pass, shifted exponentials and their sum
                p = np.where(ok, np.exp(s - m[:, None]), 0.0)
                l = p.sum(axis=1)
                # step 5: normalised weighted sum of values and the log-sum-exp
                o = (p @ Vb) / np.where(any_ok, l, 1.0)[:, None]
                O[b, h, r0:r0 + len(idx)] = np.where(any_ok[:, None], o, 0.0)
                LSE[b, h, r0:r0 + len(idx)] = np.where(any_ok, m + np.log(np.where(any_ok, l, 1.0)), -np.inf)
    return O, LSE


def online_ref(q, k, v, scale: float, tiles: Sequence[int], causal: bool = False,
               seqlen: Optional[int] = None):
    """One head, key blocks of the given sizes, running (m, l, a) carried across blocks.

    This follows the update of [CSW] "How can softmax be computed across tiles?":
    for each new block, m_new = max(m, block max); the old statistics are rescaled by
    exp(m - m_new); l gains the block's sum of exp(s - m_new) and a gains the same
    weights times the block's values; the output is a / l.  A block holding no key
    the row may see adds nothing.  ``tiles`` partitions the N keys (sizes sum to N).

    q, k, v : [N, d] (one head).  Returns (O [N, d], LSE [N]) in float64 and, for
    inspection, the per-row list of (m, l, a) after every block.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    N = q.shape[0]
    Nk = k.shape[0]
    d = v.shape[1]
    if sum(tiles) != Nk or any(t <= 0 for t in tiles):
        raise ValueError("tiles must be positive sizes summing to the number of keys")
    L = Nk if seqlen is None else int(min(max(seqlen, 0), Nk))
    c = float(scale)
    O = np.zeros((N, d))
    LSE = np.full(N, -np.inf)
    history = []
    for i in range(N):
        m = -np.inf
        l = 0.0
        a = np.zeros(d)
        hist_i = []
        j0 = 0
        for t in tiles:
            js = np.arange(j0, j0 + t)
            j0 += t
            vis = js < L
            if causal:
                vis &= js <= i
            if not vis.any():
                hist_i.append((m, l, a.copy()))
                continue
            s = (k[js[vis]] @ q[i]) * c
            m_new = max(m, float(s.max()))
            rescale = math.exp(m - m_new)      # exp(-inf) = 0 before the first visible key
            w = np.exp(s - m_new)
            l = rescale * l + float(w.sum())
            a = rescale * a + w @ v[js[vis]]
            m = m_new
            hist_i.append((m, l, a.copy()))
        history.append(hist_i)
        if l > 0.0:
            O[i] = a / l
            LSE[i] = m + math.log(l)
    return O, LSE, history


def brute_ref(q, k, v, scale: float, causal: bool = False, seqlen: Optional[int] = None):
    """Pure-Python triple loop with exactly rounded sums (``math.fsum``); tiny inputs only.

    q, k, v : nested lists or arrays [N, d] for one head.  Returns (O, LSE) as lists.
    """
    q = [[float(x) for x in row] for row in q]
    k = [[float(x) for x in row] for row in k]
    v = [[float(x) for x in row] for row in v]
    N, Nk, d = len(q), len(k), len(v[0])
    L = Nk if seqlen is None else min(max(int(seqlen), 0), Nk)
    O, LSE = [], []
    for i in range(N):
        vis = [j for j in range(Nk) if j < L and (not causal or j <= i)]
        if not vis:
            O.append([0.0] * d)
            LSE.append(-math.inf)
            continue
        s = {j: scale * math.fsum(q[i][t] * k[j][t] for t in range(d)) for j in vis}
        mx = max(s.values())
        e = {j: math.exp(s[j] - mx) for j in vis}
        den = math.fsum(e.values())
        O.append([math.fsum(e[j] * v[j][t] for j in vis) / den for t in range(d)])
        LSE.append(mx + math.log(den))
    return O, LSE


def softmax_weights_ref(q, k, scale: float, causal: bool = False, seqlen: Optional[int] = None):
    """Row-softmax weights [N, Nk] of one head (float64), visible keys only; rows with
    no visible key are all zero.  Same arithmetic as ``attention_ref`` before the V product."""
    q = _as_f64(q)
    k = _as_f64(k)
    N = q.shape[0]
    Nk = k.shape[0]
    L = Nk if seqlen is None else int(min(max(seqlen, 0), Nk))
    s = (q @ k.T) * float(scale)
    ok = visible_keys(np.arange(N), L, causal, Nk)
    s = np.where(ok, s, -np.inf)
    any_ok = ok.any(axis=1)
    m = np.where(any_ok, s.max(axis=1, initial=-np.inf), 0.0)
    p = np.where(ok, np.exp(s - m[:, None]), 0.0)
    l = p.sum(axis=1)
    return p / np.where(any_ok, l, 1.0)[:, None]
