"""CPU tests: the 8-bit-input oracle against the OCP E4M3 format, a library decoder and the
pages' worked example.

1. Every pin in ``oracle_fp8_pins.PINS`` passes on the real oracle.
2. Mutation check: plausible mistakes planted in a copy of the 8-bit module (wrong exponent
   bias, wrong subnormal exponent, implicit one dropped, one NaN code missed, wrong sign bit,
   a descale applied to the wrong tensor) must each fail at least one pin.
"""

import os
import types

import pytest

import oracle
from oracle import attention as fwd
from tests import oracle_fp8_pins

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")
IMPORT = "from .attention import attention_ref\n"


@pytest.mark.parametrize("pin", oracle_fp8_pins.PINS, ids=lambda p: p.__name__)
def test_pin_real_oracle(pin):
    pin(oracle)


MUTANTS = [
    ("(e - 7).astype", "(e - 8).astype", "exponent bias 8"),
    ("sub = np.ldexp(m / 8.0, -6)", "sub = np.ldexp(m / 8.0, -7)", "subnormal exponent off by one"),
    ("np.ldexp(1.0 + m / 8.0,", "np.ldexp(m / 8.0 + 0.5,", "implicit one replaced"),
    ("(c & 0x7F) == 0x7F", "c == 0x7F", "negative NaN code decoded as a number"),
    ("np.where((c >> 7) & 1, -1.0, 1.0)", "np.where((c >> 6) & 1, -1.0, 1.0)", "wrong sign bit"),
    ("    k = dequantize(k8, descale_k)", "    k = dequantize(k8, descale_v)", "key descale taken from V"),
    ("    v = dequantize(v8, descale_v)", "    v = e4m3_decode(v8)", "value descale dropped"),
]


def _load_mutant(old, new):
    with open(os.path.join(ORACLE_DIR, "attention_fp8.py")) as fh:
        src = fh.read()
    assert src.count(IMPORT) == 1
    src = src.replace(IMPORT, "")
    assert src.count(old) == 1, f"mutation anchor not unique/found: {old!r}"
    src = src.replace(old, new)
    mod = types.ModuleType("oracle_mutant_attention_fp8")
    mod.__dict__.update(attention_ref=fwd.attention_ref)
    exec(compile(src, "oracle_mutant_attention_fp8", "exec"), mod.__dict__)
    return types.SimpleNamespace(attention_ref=fwd.attention_ref, e4m3_decode=mod.e4m3_decode,
                                 attention_fp8_ref=mod.attention_fp8_ref)


@pytest.mark.parametrize("old,new,what", MUTANTS, ids=[m[2] for m in MUTANTS])
def test_planted_mistake_is_caught(old, new, what):
    impl = _load_mutant(old, new)
    failed = []
    for pin in oracle_fp8_pins.PINS:
        try:
            pin(impl)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"planted mistake '{what}' passed every pin"
