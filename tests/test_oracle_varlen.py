"""CPU tests: the fp64 packed variable-length oracle against what the pages and the mathematics fix.

1. Every pin in ``oracle_varlen_pins.PINS`` passes on the real oracle.
2. Mutation check: plausible mistakes planted in a copy of the variable-length oracle's source
   (the alignment offset with the wrong sign or left out, a strict inequality, keys taken from
   the query offsets, sequences that see their predecessors' keys, one head's keys used for
   all ...) must each fail at least one pin.
"""

import os
import types

import numpy as np
import pytest

import oracle
from oracle import attention as fwd
from tests import oracle_varlen_pins

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")
IMPORT_LINE = "from .attention import _as_f64\n"


@pytest.mark.parametrize("pin", oracle_varlen_pins.PINS, ids=lambda p: p.__name__)
def test_pin_real_oracle(pin):
    pin(oracle)


# (text to replace, replacement, what the mistake is)
MUTANTS = [
    ('        return Lk - Lq\n', '        return Lq - Lk\n', "bottom-right offset with the wrong sign"),
    ('        return Lk - Lq\n', '        return 0\n', "alignment ignored (always top-left)"),
    ('            ok = j <= i + causal_offset(Lq, Lk, align)', '            ok = j < i + causal_offset(Lq, Lk, align)',
     "causal mask hides the diagonal"),
    ('            s = np.where(ok, (q[qs:qe, h] @ k[ks:ke, h].T) * c, -np.inf)',
     '            s = np.where(ok, (q[qs:qe, h] @ k[qs:qs + Lk, h].T) * c, -np.inf)', "keys located with the query offsets"),
    ('            o = (p @ v[ks:ke, h]) / np.where(any_ok, l, 1.0)[:, None]',
     '            o = (p @ v[ks:ke, 0]) / np.where(any_ok, l, 1.0)[:, None]', "head 0's values used for every head"),
    ('            s = np.where(ok, (q[qs:qe, h] @ k[ks:ke, h].T) * c, -np.inf)',
     '            s = np.where(ok, (q[qs:qe, h] @ k[ks:ke, h].T), -np.inf)', "scale dropped"),
    ('            o = (p @ v[ks:ke, h]) / np.where(any_ok, l, 1.0)[:, None]',
     '            o = (p @ v[ks:ke, h])', "output not normalised"),
    ('            LSE[h, qs:qe] = np.where(any_ok, m + np.log(np.where(any_ok, l, 1.0)), -np.inf)',
     '            LSE[h, qs:qe] = np.where(any_ok, m, -np.inf)', "log-sum-exp misses ln l"),
    ('        Lq, Lk = qe - qs, ke - ks\n', '        ks = 0\n        Lq, Lk = qe - qs, ke - ks\n',
     "each sequence also sees its predecessors' keys"),
]


def _load_mutant(old, new):
    with open(os.path.join(ORACLE_DIR, "attention_varlen.py")) as fh:
        src = fh.read()
    assert src.count(IMPORT_LINE) == 1
    src = src.replace(IMPORT_LINE, "")
    assert src.count(old) == 1, f"mutation anchor not unique/found: {old!r}"
    src = src.replace(old, new)
    mod = types.ModuleType("oracle_mutant_attention_varlen")
    mod.__dict__.update(_as_f64=fwd._as_f64)
    exec(compile(src, "oracle_mutant_attention_varlen", "exec"), mod.__dict__)
    return types.SimpleNamespace(attention_ref=fwd.attention_ref, attention_varlen_ref=mod.attention_varlen_ref,
                                 brute_varlen_ref=mod.brute_varlen_ref)


@pytest.mark.parametrize("mut", MUTANTS, ids=[m[2] for m in MUTANTS])
def test_mutant_is_caught(mut):
    old, new, _ = mut
    impl = _load_mutant(old, new)
    failed = []
    with np.errstate(all="ignore"):
        for pin in oracle_varlen_pins.PINS:
            try:
                pin(impl)
            except Exception as e:  # AssertionError or a crash both count as caught
                failed.append((pin.__name__, type(e).__name__))
    assert failed, "no pin catches this planted mistake"


def test_unmutated_copy_passes_all_pins():
    impl = _load_mutant("        return Lk - Lq\n", "        return Lk - Lq\n")
    for pin in oracle_varlen_pins.PINS:
        pin(impl)
