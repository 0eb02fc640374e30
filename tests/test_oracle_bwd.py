"""CPU tests: the fp64 attention-gradient oracle against what the pages and the mathematics fix.

1. Every pin in ``oracle_bwd_pins.PINS`` passes on the real oracle.
2. Mutation check: plausible mistakes planted in a copy of the gradient oracle's source (a
   dropped softmax row term, a missing transpose, a missing scale, a wrong sign ...) must each
   fail at least one pin.
"""

import os
import types

import numpy as np
import pytest

import oracle
from oracle import attention as fwd
from tests import oracle_bwd_pins

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")
IMPORT_LINE = "from .attention import _as_f64, visible_keys\n"


@pytest.mark.parametrize("pin", oracle_bwd_pins.PINS, ids=lambda p: p.__name__)
def test_pin_real_oracle(pin):
    pin(oracle)


# (text to replace, replacement, what the mistake is)
MUTANTS = [
    ("            dV[b, h] = P.T @ G", "            dV[b, h] = P @ G", "value gradient without the transpose"),
    ("            dS = P * (dP - row[:, None])", "            dS = P * dP", "softmax row term dropped"),
    ("            dS = P * (dP - row[:, None])", "            dS = P * (dP + row[:, None])", "row term with the wrong sign"),
    ("            dS = P * (dP - row[:, None])", "            dS = dP - row[:, None]", "probability factor dropped"),
    ("            row = (P * dP).sum(axis=1)", "            row = (P * dP).sum(axis=0)", "row term summed over keys' axis"),
    ("            dQ[b, h] = c * (dS @ K)", "            dQ[b, h] = dS @ K", "query gradient misses the scale"),
    ("            dK[b, h] = c * (dS.T @ Q)", "            dK[b, h] = c * (dS @ Q)", "key gradient without the transpose"),
    ("            dK[b, h] = c * (dS.T @ Q)", "            dK[b, h] = -c * (dS.T @ Q)", "key gradient with the wrong sign"),
    ("            dP = G @ V.T", "            dP = G @ V[::-1].T", "value rows out of order in dP"),
    ("            P = e / np.where(any_ok, den, 1.0)[:, None]", "            P = e", "probabilities unnormalised"),
    ("        ok = visible_keys(np.arange(N), L, causal, Nk)", "        ok = visible_keys(np.arange(N), Nk, causal, Nk)",
     "key padding ignored"),
    ("    return (o * do).sum(axis=-1)", "    return (o * do).sum(axis=-2)", "row term over the wrong axis"),
]


def _load_mutant(old, new):
    with open(os.path.join(ORACLE_DIR, "attention_bwd.py")) as fh:
        src = fh.read()
    assert src.count(IMPORT_LINE) == 1
    src = src.replace(IMPORT_LINE, "")
    assert src.count(old) == 1, f"mutation anchor not unique/found: {old!r}"
    src = src.replace(old, new)
    mod = types.ModuleType("oracle_mutant_attention_bwd")
    mod.__dict__.update(_as_f64=fwd._as_f64, visible_keys=fwd.visible_keys)
    exec(compile(src, "oracle_mutant_attention_bwd", "exec"), mod.__dict__)
    return types.SimpleNamespace(attention_ref=fwd.attention_ref, softmax_weights_ref=fwd.softmax_weights_ref,
                                 attention_bwd_ref=mod.attention_bwd_ref, row_dot_ref=mod.row_dot_ref)


@pytest.mark.parametrize("mut", MUTANTS, ids=[m[2] for m in MUTANTS])
def test_mutant_is_caught(mut):
    old, new, _ = mut
    impl = _load_mutant(old, new)
    failed = []
    with np.errstate(all="ignore"):
        for pin in oracle_bwd_pins.PINS:
            try:
                pin(impl)
            except Exception as e:  # AssertionError or a crash both count as caught
                failed.append((pin.__name__, type(e).__name__))
    assert failed, "no pin catches this planted mistake"


def test_unmutated_copy_passes_all_pins():
    impl = _load_mutant("    return (o * do).sum(axis=-1)", "    return (o * do).sum(axis=-1)")
    for pin in oracle_bwd_pins.PINS:
        pin(impl)
