"""Pins of the 8-bit-input oracle: the OCP E4M3 format's fixed points, a library decoder, and
what the mathematics fixes.

Each pin takes an ``impl`` namespace (the oracle package, or a mutant of the 8-bit module) and
raises on a mismatch.

* Fixed points of the format: 0x38 = 1, 0x40 = 2, 0x30 = 1/2, 0x7E = 448 (largest finite),
  0x08 = 2^-6 (smallest normal), 0x07 = 7/8 * 2^-6 (largest subnormal), 0x01 = 2^-9, signed
  zeros, NaN at 0x7F and 0xFF.
* All 256 codes agree with PyTorch's float8_e4m3fn decoding (a library routine).
* The finite positive codes increase strictly; a set sign bit negates.
* The pages' two-key worked example, carried in 8-bit codes with a key descale of ln 3: output
  5 and log-sum-exp ln 4.
* Descales: doubling the Q or K descale equals doubling the score scale; the V descale
  multiplies O and leaves the log-sum-exp alone; with unit descales the oracle equals the
  float oracle on the library-decoded inputs.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _codes(seed, shape):
    """Random finite E4M3 codes (NaN codes 0x7F / 0xFF replaced by 0x00)."""
    c = np.random.default_rng(seed).integers(0, 256, size=shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0
    return c


def pin_fixed_points(impl):
    dec = impl.e4m3_decode
    want = {0x38: 1.0, 0x40: 2.0, 0x30: 0.5, 0x7E: 448.0, 0xFE: -448.0, 0x08: 2.0 ** -6,
            0x07: 7.0 / 8.0 * 2.0 ** -6, 0x01: 2.0 ** -9, 0x81: -(2.0 ** -9), 0x4C: 6.0, 0x00: 0.0}
    got = dec(np.array(list(want), dtype=np.uint8))
    for (c, w), g in zip(want.items(), got):
        assert g == w, (hex(c), g, w)
    z = dec(np.array([0x00, 0x80], dtype=np.uint8))
    assert z[0] == 0 and not math.copysign(1.0, z[0]) < 0 and math.copysign(1.0, z[1]) < 0
    nan = dec(np.array([0x7F, 0xFF], dtype=np.uint8))
    assert np.isnan(nan).all(), nan


def pin_matches_library_decoder(impl):
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = impl.e4m3_decode(codes)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), [hex(c) for c in codes[~same]]


def pin_monotone_and_sign(impl):
    pos = impl.e4m3_decode(np.arange(0x00, 0x7F, dtype=np.uint8))
    assert (np.diff(pos) > 0).all()
    neg = impl.e4m3_decode(np.arange(0x80, 0xFF, dtype=np.uint8))
    assert np.array_equal(neg, -pos)


def pin_two_key_example(impl):
    """[CSW] "How can softmax be computed across tiles?": scores 0 and ln 3 with values 2 and 6
    give output 5 (weights 1/4, 3/4) and l = 4.  The key codes are (0, 1) and (1, 1) with a
    key descale of ln 3, so the scores are 0 and ln 3 up to the float32 rounding of ln 3."""
    with open(os.path.join(GOLDEN, "two_tile_example.json")) as f:
        g = json.load(f)
    q8 = np.array([[0x38, 0x00]], dtype=np.uint8)[None, None]          # (1, 0)
    k8 = np.array([[0x00, 0x38], [0x38, 0x38]], dtype=np.uint8)[None, None]
    v8 = np.array([[0x40, 0x38], [0x4C, 0x38]], dtype=np.uint8)[None, None]   # (2, 1), (6, 1)
    dk = float(np.float32(g["tile_scores"][1]))
    O, L = impl.attention_fp8_ref(q8, k8, v8, 1.0, dk, 1.0, 1.0)
    assert abs(O[0, 0, 0, 0] - g["output"]) < 1e-6, O[0, 0, 0, 0]
    assert abs(O[0, 0, 0, 1] - 1.0) < 1e-15
    assert abs(L[0, 0, 0] - math.log(4.0)) < 1e-7, L[0, 0, 0]


def pin_descales(impl):
    q8, k8, v8 = (_codes(s, (1, 2, 7, 8)) for s in (1, 2, 3))
    # codes up to 448 make huge logits: keep the scale small so rows are not one-hot
    s = 1e-3
    base_o, base_l = impl.attention_fp8_ref(q8, k8, v8, 1.0, 1.0, 1.0, 2 * s, causal=True)
    for dq, dk in ((2.0, 1.0), (1.0, 2.0)):
        o, l = impl.attention_fp8_ref(q8, k8, v8, dq, dk, 1.0, s, causal=True)
        assert np.allclose(o, base_o, rtol=1e-12, atol=1e-12) and np.allclose(l, base_l, rtol=1e-12, atol=1e-12)
    o, l = impl.attention_fp8_ref(q8, k8, v8, 1.0, 1.0, 0.375, 2 * s, causal=True)
    assert np.allclose(o, 0.375 * base_o, rtol=1e-12, atol=1e-12)
    assert np.array_equal(l, base_l)


def pin_reduces_to_float_oracle(impl):
    import torch
    q8, k8, v8 = (_codes(s, (2, 1, 9, 4)) for s in (4, 5, 6))
    dec = [torch.from_numpy(x.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy() for x in (q8, k8, v8)]
    dq, dk, dv = 0.01, 0.02, 0.5
    o, l = impl.attention_fp8_ref(q8, k8, v8, dq, dk, dv, 0.25, seqlens=[5, 0])
    ro, rl = impl.attention_ref(np.float32(dq) * dec[0], np.float32(dk) * dec[1], np.float32(dv) * dec[2], 0.25,
                                seqlens=[5, 0])
    assert np.allclose(o, ro, rtol=1e-13, atol=1e-13)
    # batch 1 has no visible key: O = 0 and LSE = -inf on both sides
    assert np.isneginf(l[1]).all() and np.isneginf(rl[1]).all() and not o[1].any()
    assert np.allclose(l[0], rl[0], rtol=1e-13, atol=0)


PINS = [pin_fixed_points, pin_matches_library_decoder, pin_monotone_and_sign, pin_two_key_example, pin_descales,
        pin_reduces_to_float_oracle]
