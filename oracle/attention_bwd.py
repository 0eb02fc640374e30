"""fp64 CPU oracle for the gradient of exact attention -- TEST INFRASTRUCTURE, not part of the product.

Only the test suite, the smoke check and the benchmark may import this module.  It shares no
code with the HIP path and imports nothing from it.

Sources (web pages, cited by title and section):

* [CSW] "FlashAttention Interview Questions: IO Complexity, Tiling, and Numerical
  Stability" (cswork.org).  Section "What is FlashAttention exact about?" fixes the
  forward target O = row_softmax(scale * Q K^T + mask) V.  Section "Why can recomputation help
  training?" explains that the backward pass needs the attention probabilities again and that
  a tiled implementation recomputes them from Q, K and the saved normalisation statistics
  rather than storing the N x N matrix.

Because the tiled backward reaches exactly the gradient of the plain definition (up to
rounding order), ``attention_bwd_ref`` is that gradient written out in float64 with the whole
probability matrix of each head materialised: no tiling, no recomputation.

Readings (also listed in the design notes):

* Only the output O receives an incoming gradient dO; the log-sum-exp is an auxiliary output
  and is not differentiated.
* Masked keys are removed from the softmax (their probability is exactly 0), so they receive
  zero gradient, and a row with no visible key contributes nothing.
* The chain rule through the row softmax: for P = softmax(S) and an upstream gradient dP of P,
  dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik).  With O = P V the upstream gradient is dP = dO V^T
  and sum_k P_ik dP_ik equals dO_i . O_i.
"""

from __future__ import annotations

import numpy as np

from .attention import _as_f64, visible_keys


def attention_bwd_ref(q, k, v, do, scale: float, causal: bool = False, seqlens=None):
    """Gradients of O = softmax(scale Q K^T, masked) V with respect to Q, K and V.

    Parameters
    ----------
    q, k, v, do : array-like [B, H, N, d]; upcast to float64 exactly.
    scale : multiplier of the dot products (the float32 value the kernel receives).
    causal : hide keys j > i.
    seqlens : optional int sequence [B]; keys j >= seqlens[b] are hidden.

    Returns
    -------
    (dQ, dK, dV) float64 [B, H, N, d].
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    do = _as_f64(do)
    B, H, N, d = q.shape
    Nk = k.shape[2]
    c = float(scale)
    dQ = np.zeros_like(q)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    for b in range(B):
        L = Nk if seqlens is None else int(min(max(int(seqlens[b]), 0), Nk))
        ok = visible_keys(np.arange(N), L, causal, Nk)          # [N, Nk]
        any_ok = ok.any(axis=1)
        for h in range(H):
            Q, K, V, G = q[b, h], k[b, h], v[b, h], do[b, h]
            # forward, materialised: probabilities of the visible keys, 0 elsewhere
            s = np.where(ok, (Q @ K.T) * c, -np.inf)
            m = np.where(any_ok, s.max(axis=1, initial=-np.inf), 0.0)
            e = np.where(ok, np.exp(s - m[:, None]), 0.0)
            den = e.sum(axis=1)
            P = e / np.where(any_ok, den, 1.0)[:, None]
            # O = P V: gradient with respect to V and to P
            dV[b, h] = P.T @ G
            dP = G @ V.T
            # row softmax: dS = P * (dP - rowsum(P * dP))
            row = (P * dP).sum(axis=1)
            dS = P * (dP - row[:, None])
            # S = scale * Q K^T
            dQ[b, h] = c * (dS @ K)
            dK[b, h] = c * (dS.T @ Q)
    return dQ, dK, dV


def row_dot_ref(o, do):
    """D_i = dO_i . O_i per row, float64 [B, H, N] (the row term of the softmax gradient)."""
    o = _as_f64(o)
    do = _as_f64(do)
    return (o * do).sum(axis=-1)
