"""CPU tests: the fp64 oracle against what the pages and the mathematics fix.

1. Every pin in ``oracle_pins.PINS`` passes on the real oracle.
2. Mutation check: plausible mistakes are planted in a *copy* of the oracle's source
   (a dropped term, a wrong sign, an off-by-one mask, a transposed operand, a missing
   rescale ...).  Each mutant must fail at least one pin, which shows the pins have the
   power to catch that mistake.
"""

import os
import types

import numpy as np
import pytest

import oracle
from oracle import accounting
from tests import oracle_pins

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda p: p.__name__)
def test_pin_real_oracle(pin):
    pin(oracle)


# (file, text to replace, replacement, what the mistake is)
MUTANTS = [
    ("attention.py", "ok = ok & (j <= np.asarray(i)[:, None])", "ok = ok & (j < np.asarray(i)[:, None])",
     "causal mask hides the diagonal"),
    ("attention.py", "ok = ok & (j <= np.asarray(i)[:, None])", "ok = ok & (j >= np.asarray(i)[:, None])",
     "causal mask reversed"),
    ("attention.py", "    ok = j < L\n", "    ok = j < max(L - 1, 0)\n", "padding hides one key too many"),
    ("attention.py", "s = (q[b, h, idx] @ Kb.T) * c", "s = (q[b, h, idx] @ Kb.T)", "scale dropped"),
    ("attention.py", "s = (q[b, h, idx] @ Kb.T) * c", "s = (q[b, h, idx] @ Kb.T) * c * c", "scale applied twice"),
    ("attention.py", "s = (q[b, h, idx] @ Kb.T) * c", "s = (Kb[:len(idx)] @ q[b, h, idx].T)[:len(idx)] * c",
     "operands swapped (keys against queries)"),
    ("attention.py", "                p = np.where(ok, np.exp(s - m[:, None]), 0.0)",
     "                p = np.where(ok, np.exp(s + m[:, None]), 0.0)",
     "wrong sign of the max shift"),
    ("attention.py", "                m = np.where(any_ok, s.max(axis=1, initial=-np.inf), 0.0)",
     "                m = np.where(any_ok, np.where(ok, s, np.inf).min(axis=1), 0.0)", "shift by the minimum, not the maximum"),
    ("attention.py", "o = (p @ Vb) / np.where(any_ok, l, 1.0)[:, None]", "o = (p @ Vb)", "normalisation dropped"),
    ("attention.py", "o = (p @ Vb) / np.where(any_ok, l, 1.0)[:, None]",
     "o = (p @ Vb[::-1]) / np.where(any_ok, l, 1.0)[:, None]", "value rows out of order"),
    ("attention.py", "m + np.log(np.where(any_ok, l, 1.0))", "np.log(np.where(any_ok, l, 1.0))",
     "LSE misses the max"),
    ("attention.py", "m + np.log(np.where(any_ok, l, 1.0))", "m + np.log2(np.where(any_ok, l, 1.0))",
     "LSE in the wrong base"),
    ("attention.py", "O[b, h, r0:r0 + len(idx)] = np.where(any_ok[:, None], o, 0.0)",
     "O[b, h, r0:r0 + len(idx)] = np.where(any_ok[:, None], o, np.nan)", "all-masked row gives NaN"),
    ("attention.py", "            Kb = k[b, h, :L]", "            Kb = k[b, (h + 1) % H, :L]", "wrong head's keys"),
    ("attention.py", "            l = rescale * l + float(w.sum())", "            l = l + float(w.sum())",
     "running sum not rescaled"),
    ("attention.py", "            a = rescale * a + w @ v[js[vis]]", "            a = a + w @ v[js[vis]]",
     "accumulator not rescaled"),
    ("attention.py", "            m_new = max(m, float(s.max()))", "            m_new = float(s.max())",
     "running max forgets earlier tiles"),
    ("attention.py", "            O[i] = a / l", "            O[i] = a", "online output not divided by l"),
    ("attention.py", "                vis &= js <= i", "                vis &= js < i", "online causal hides the diagonal"),
    ("attention.py", "        vis = [j for j in range(Nk) if j < L and (not causal or j <= i)]",
     "        vis = [j for j in range(Nk) if j < L and (not causal or j < i)]", "brute-force causal off by one"),
    ("attention.py", "        LSE.append(mx + math.log(den))", "        LSE.append(math.log(den))",
     "brute-force LSE misses the max"),
    ("attention.py", "    return p / np.where(any_ok, l, 1.0)[:, None]", "    return p", "weights unnormalised"),
    ("accounting.py", "    return N * N\n", "    return N * (N - 1)\n", "score count off by one row"),
    ("accounting.py", "    return 4 * head_tensor_bytes(N, d, elem_bytes)", "    return 3 * head_tensor_bytes(N, d, elem_bytes)",
     "output tensor left out"),
]


def _load_mutant(fname, old, new):
    srcs = {}
    for f in ("attention.py", "accounting.py"):
        with open(os.path.join(ORACLE_DIR, f)) as fh:
            srcs[f] = fh.read()
    assert srcs[fname].count(old) == 1, f"mutation anchor not unique/found: {old!r}"
    srcs[fname] = srcs[fname].replace(old, new)
    att = types.ModuleType("oracle_mutant_attention")
    exec(compile(srcs["attention.py"], "oracle_mutant_attention", "exec"), att.__dict__)
    acc = types.ModuleType("oracle_mutant_accounting")
    exec(compile(srcs["accounting.py"], "oracle_mutant_accounting", "exec"), acc.__dict__)
    return types.SimpleNamespace(attention_ref=att.attention_ref, online_ref=att.online_ref,
                                 brute_ref=att.brute_ref, softmax_weights_ref=att.softmax_weights_ref,
                                 accounting=acc)


@pytest.mark.parametrize("mut", MUTANTS, ids=[m[3] for m in MUTANTS])
def test_mutant_is_caught(mut):
    fname, old, new, _ = mut
    impl = _load_mutant(fname, old, new)
    failed = []
    with np.errstate(all="ignore"):
        for pin in oracle_pins.PINS:
            try:
                pin(impl)
            except Exception as e:  # AssertionError or a crash both count as caught
                failed.append((pin.__name__, type(e).__name__))
    assert failed, "no pin catches this planted mistake"


def test_unmutated_copy_passes_all_pins():
    """The mutation loader itself must not break a correct oracle."""
    impl = _load_mutant("accounting.py", "MIB = 1 << 20", "MIB = 1 << 20")
    for pin in oracle_pins.PINS:
        pin(impl)


def test_accounting_module_is_oracle_module():
    assert oracle.accounting is accounting
