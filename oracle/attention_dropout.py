"""fp64 CPU oracle for exact attention with dropout on the probabilities -- TEST INFRASTRUCTURE,
not part of the product.

Only the test suite, the smoke check and the benchmark may import this module.  It shares no
code with the HIP path and imports nothing from it.

Sources (web pages, cited by title and section):

* [CSW] "FlashAttention Interview Questions: IO Complexity, Tiling, and Numerical Stability"
  (cswork.org), section "Does subtracting the maximum solve every numerical issue?": dropout is
  first disabled for correctness tests, then its enabled behaviour is tested against the
  implementation's random-number and reproducibility contract.  Section "What is FlashAttention
  exact about?" fixes the attention being dropped out.

The pages give no contract, so this module defines one (also listed in the design notes):

* Dropout acts on the normalised probabilities: O = (P * Z) V with P = softmax(scale Q K^T over
  visible keys) and Z_ij = keep_ij / (1 - p_eff).  The log-sum-exp is that of P, before dropout.
* Random numbers: Philox4x32-10 (``oracle.philox``) under the 64-bit key `seed`.  Element
  (b, h, i, j) -- query row i, key j of head h of batch element b, bh = b * H + h -- takes byte
  4 * (i mod 4) + (j mod 4) of the 16 output bytes (little-endian words) of the counter
  (j div 4, i div 4, bh, offset).  Every 4 x 4 block of (row, key) pairs thus comes from one
  Philox call and no two elements share a byte.
* The drop probability is quantised to 1/256: t = round(256 p) (0 <= t <= 255), an element is
  kept iff its byte >= t, and p_eff = t / 256.
* Gradients follow the chain rule through O = (P * Z) V with Z fixed: dV = (P * Z)^T dO,
  dP = Z * (dO V^T), D_i = sum_j P_ij dP_ij (= dO_i . O_i), dS = P * (dP - D),
  dQ = scale dS K, dK = scale dS^T Q.
"""

from __future__ import annotations

import numpy as np

from .attention import _as_f64, attention_ref, softmax_weights_ref
from .philox import M0, M1, W0, W1, philox4x32


def dropout_threshold(p: float) -> int:
    """t = round(256 p), the byte threshold of the contract (0 <= p < 255.5 / 256)."""
    t = int(np.floor(256.0 * float(p) + 0.5))
    if not 0 <= t <= 255:
        raise ValueError("drop probability must lie in [0, 255.5/256)")
    return t


def _philox_np(c0, c1, c2, c3, k0, k1, rounds=10):
    """Philox4x32 on arrays of counters (uint64 holding 32-bit values), one key."""
    m = np.uint64(0xFFFFFFFF)
    c0, c1, c2, c3 = (np.asarray(x, dtype=np.uint64) & m for x in (c0, c1, c2, c3))
    k0, k1 = np.uint64(k0 & 0xFFFFFFFF), np.uint64(k1 & 0xFFFFFFFF)
    for _ in range(rounds):
        p0 = np.uint64(M0) * c0
        p1 = np.uint64(M1) * c2
        c0, c1, c2, c3 = ((p1 >> np.uint64(32)) ^ c1 ^ k0) & m, p1 & m, ((p0 >> np.uint64(32)) ^ c3 ^ k1) & m, p0 & m
        k0 = (k0 + np.uint64(W0)) & m
        k1 = (k1 + np.uint64(W1)) & m
    return c0, c1, c2, c3


def keep_mask(bh: int, n_rows: int, n_keys: int, seed: int, offset: int, p: float) -> np.ndarray:
    """Boolean [n_rows, n_keys]: is element (i, j) of head bh kept?  (vectorised contract)"""
    t = dropout_threshold(p)
    i = np.arange(n_rows)[:, None]
    j = np.arange(n_keys)[None, :]
    j4 = np.broadcast_to(j // 4, (n_rows, n_keys))
    i4 = np.broadcast_to(i // 4, (n_rows, n_keys))
    words = _philox_np(j4, i4, np.full_like(j4, bh), np.full_like(j4, offset & 0xFFFFFFFF),
                       seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    w = np.stack(words, axis=0)                                   # [4, rows, keys]
    word = np.take_along_axis(w, np.broadcast_to(i % 4, (n_rows, n_keys))[None], axis=0)[0]
    byte = (word >> (np.uint64(8) * np.broadcast_to(j % 4, (n_rows, n_keys)).astype(np.uint64))) & np.uint64(0xFF)
    return byte >= np.uint64(t)


def keep_mask_loop(bh: int, n_rows: int, n_keys: int, seed: int, offset: int, p: float):
    """The same contract element by element with the pure-Python Philox; tiny sizes only."""
    t = dropout_threshold(p)
    out = np.zeros((n_rows, n_keys), dtype=bool)
    for i in range(n_rows):
        for j in range(n_keys):
            words = philox4x32((j // 4, i // 4, bh, offset), (seed, seed >> 32))
            out[i, j] = ((words[i % 4] >> (8 * (j % 4))) & 0xFF) >= t
    return out


def attention_dropout_ref(q, k, v, scale: float, p: float, seed: int, offset: int, causal: bool = False,
                          seqlens=None):
    """(O, LSE) of attention with dropout on the probabilities, float64; [B, H, N, d] inputs."""
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    B, H, N, _ = q.shape
    Nk = k.shape[2]
    keep_scale = 256.0 / (256 - dropout_threshold(p))
    _, LSE = attention_ref(q, k, v, scale, causal=causal, seqlens=seqlens)   # before dropout
    O = np.zeros((B, H, N, v.shape[3]))
    for b in range(B):
        L = Nk if seqlens is None else int(min(max(int(seqlens[b]), 0), Nk))
        for h in range(H):
            P = softmax_weights_ref(q[b, h], k[b, h], scale, causal=causal, seqlen=L)
            Z = keep_mask(b * H + h, N, Nk, seed, offset, p) * keep_scale
            O[b, h] = (P * Z) @ v[b, h]
    return O, LSE


def attention_dropout_bwd_ref(q, k, v, do, scale: float, p: float, seed: int, offset: int, causal: bool = False,
                              seqlens=None):
    """(dQ, dK, dV) of O = (P * Z) V with the contract's fixed Z, float64."""
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    do = _as_f64(do)
    B, H, N, _ = q.shape
    Nk = k.shape[2]
    keep_scale = 256.0 / (256 - dropout_threshold(p))
    c = float(scale)
    dQ, dK, dV = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        L = Nk if seqlens is None else int(min(max(int(seqlens[b]), 0), Nk))
        for h in range(H):
            P = softmax_weights_ref(q[b, h], k[b, h], scale, causal=causal, seqlen=L)
            Z = keep_mask(b * H + h, N, Nk, seed, offset, p) * keep_scale
            G = do[b, h]
            dV[b, h] = (P * Z).T @ G
            dP = Z * (G @ v[b, h].T)
            row = (P * dP).sum(axis=1)
            dS = P * (dP - row[:, None])
            dQ[b, h] = c * (dS @ k[b, h])
            dK[b, h] = c * (dS.T @ q[b, h])
    return dQ, dK, dV
