"""CPU tests: the dropout oracle and its Philox generator against what is published and what the
mathematics fixes.

1. Every pin in ``oracle_dropout_pins.PINS`` passes on the real oracle.
2. Mutation check: plausible mistakes planted in a copy of the dropout module (the keep scale
   left out, counter words swapped, the wrong byte, a strict threshold, the mask left out of a
   gradient product, a floored threshold ...) must each fail at least one pin.
"""

import os
import types

import numpy as np
import pytest

import oracle
from oracle import attention as fwd
from oracle import philox as ph
from tests import oracle_dropout_pins

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")
IMPORTS = ["from .attention import _as_f64, attention_ref, softmax_weights_ref\n",
           "from .philox import M0, M1, W0, W1, philox4x32\n"]


@pytest.mark.parametrize("pin", oracle_dropout_pins.PINS, ids=lambda p: p.__name__)
def test_pin_real_oracle(pin):
    pin(oracle)


MUTANTS = [
    ("    keep_scale = 256.0 / (256 - dropout_threshold(p))\n    _, LSE", "    keep_scale = 1.0\n    _, LSE",
     "kept probabilities not rescaled"),
    ("    words = _philox_np(j4, i4, np.full_like(j4, bh)", "    words = _philox_np(i4, j4, np.full_like(j4, bh)",
     "counter words swapped"),
    ("np.broadcast_to(i % 4, (n_rows, n_keys))[None]", "np.broadcast_to(j % 4, (n_rows, n_keys))[None]",
     "word chosen by the key instead of the row"),
    ("    return byte >= np.uint64(t)", "    return byte > np.uint64(t)", "strict threshold"),
    ("            dV[b, h] = (P * Z).T @ G", "            dV[b, h] = P.T @ G", "value gradient ignores the mask"),
    ("            dP = Z * (G @ v[b, h].T)", "            dP = G @ v[b, h].T", "probability gradient ignores the mask"),
    ("    t = int(np.floor(256.0 * float(p) + 0.5))", "    t = int(np.floor(256.0 * float(p)))", "threshold floored"),
    ("        k0 = (k0 + np.uint64(W0)) & m", "        k0 = (k0 + np.uint64(W1)) & m", "wrong Weyl constant"),
]


def _load_mutant(old, new):
    with open(os.path.join(ORACLE_DIR, "attention_dropout.py")) as fh:
        src = fh.read()
    for line in IMPORTS:
        assert src.count(line) == 1, line
        src = src.replace(line, "")
    assert src.count(old) == 1, f"mutation anchor not unique/found: {old!r}"
    src = src.replace(old, new)
    mod = types.ModuleType("oracle_mutant_attention_dropout")
    mod.__dict__.update(_as_f64=fwd._as_f64, attention_ref=fwd.attention_ref,
                        softmax_weights_ref=fwd.softmax_weights_ref, M0=ph.M0, M1=ph.M1, W0=ph.W0, W1=ph.W1,
                        philox4x32=ph.philox4x32)
    exec(compile(src, "oracle_mutant_attention_dropout", "exec"), mod.__dict__)
    return types.SimpleNamespace(attention_ref=fwd.attention_ref, philox4x32=ph.philox4x32,
                                 **{n: getattr(mod, n) for n in ("attention_dropout_ref", "attention_dropout_bwd_ref",
                                                                 "dropout_threshold", "keep_mask", "keep_mask_loop",
                                                                 "_philox_np")})


@pytest.mark.parametrize("mut", MUTANTS, ids=[m[2] for m in MUTANTS])
def test_mutant_is_caught(mut):
    old, new, _ = mut
    impl = _load_mutant(old, new)
    failed = []
    with np.errstate(all="ignore"):
        for pin in oracle_dropout_pins.PINS:
            try:
                pin(impl)
            except Exception as e:  # AssertionError or a crash both count as caught
                failed.append((pin.__name__, type(e).__name__))
    assert failed, "no pin catches this planted mistake"


def test_unmutated_copy_passes_all_pins():
    impl = _load_mutant("    return byte >= np.uint64(t)", "    return byte >= np.uint64(t)")
    for pin in oracle_dropout_pins.PINS:
        pin(impl)
