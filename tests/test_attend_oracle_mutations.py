"""Plants plausible mistakes in a copy of the attention oracle (on the CPU) and checks that the
pins in test_attend_oracle_pins.py catch every one of them."""
import inspect
import sys
import types

import pytest

import oracle.attend_oracle as ao

from . import test_attend_oracle_pins as pins

SRC = inspect.getsource(ao)

MUTATIONS = {
    "scale dropped": ("        z = scale * (K @ q[g])\n", "        z = K @ q[g]\n"),
    "no max shift": ("        z = z - z.max()\n", "        z = z\n"),
    "keys and values swapped": ("    K = rebuild(Dk, k_idx, k_coef)\n    V = rebuild(Dv, v_idx, v_coef)",
                                "    K = rebuild(Dv, v_idx, v_coef)\n    V = rebuild(Dk, k_idx, k_coef)"),
    "one token too few": ("        L = int(lens[r])\n", "        L = max(int(lens[r]) - 1, 0)\n"),
    "empty slots counted": ("            if 0 <= j < D.shape[0]:", "            if j < D.shape[0]:"),
    "first slot skipped": ("        for k in range(s):\n            j = int(idx[t, k])",
                           "        for k in range(1, s):\n            j = int(idx[t, k])"),
    "unnormalised weights": ("        p = p / p.sum()\n", "        p = p / len(p)\n"),
}


def _run_pins():
    failed = []
    for name, f in sorted(vars(pins).items()):
        if not name.startswith("test_") or not callable(f):
            continue
        params = [()]
        if name == "test_softmax_is_shift_invariant_and_overflow_safe":
            params = [(0.0,), (800.0,)]
        for args in params:
            try:
                f(*args)
            except Exception:
                failed.append(name)
    return failed


def _mutant(old, new):
    assert SRC.count(old) == 1, f"mutation text matches {SRC.count(old)} times"
    mod = types.ModuleType("attend_oracle_mutant")
    sys.modules["attend_oracle_mutant"] = mod
    try:
        exec(compile(SRC.replace(old, new), "attend_oracle_mutant", "exec"), mod.__dict__)
    finally:
        del sys.modules["attend_oracle_mutant"]
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name, monkeypatch):
    monkeypatch.setattr(pins, "ao", _mutant(*MUTATIONS[name]))
    assert _run_pins(), f"no pin caught mutation {name!r}"


def test_unmutated_copy_passes_every_pin(monkeypatch):
    monkeypatch.setattr(pins, "ao", _mutant("import numpy as np\n", "import numpy as np\n"))
    assert _run_pins() == []
