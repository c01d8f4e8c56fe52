"""Plants plausible mistakes in a copy of the oracle (on the CPU) and checks that the pins in
test_oracle_pins.py catch every one of them.

Each mutation is a literal text edit of oracle/fadkv_oracle.py applied to an in-memory copy;
the mutated module replaces the oracle's public names while the pins run, then everything is
restored.  A mutation whose text no longer matches fails loudly, so the list stays in step with
the oracle.
"""
import inspect
import sys
import types

import pytest

import oracle
import oracle.fadkv_oracle as ofk

from . import test_oracle_pins as pins

SRC = inspect.getsource(ofk)

MUTATIONS = {
    "ridge drops the absolute term":
        ("return G_SS + np.diag(ridge_abs + ridge_rel * np.diag(G_SS))",
         "return G_SS + np.diag(ridge_rel * np.diag(G_SS))"),
    "ridge ignores diag(G)":
        ("return G_SS + np.diag(ridge_abs + ridge_rel * np.diag(G_SS))",
         "return G_SS + np.diag(ridge_abs + ridge_rel * np.ones(len(G_SS)))"),
    "pool ranks signed scores":
        ("    a = np.abs(sigma)\n    order = np.lexsort((np.arange(N), -a))   # primary",
         "    a = sigma\n    order = np.lexsort((np.arange(N), -a))   # primary"),
    "pool ties to highest index":
        ("order = np.lexsort((np.arange(N), -a))   # primary key -|sigma|, then index",
         "order = np.lexsort((-np.arange(N), -a))   # primary key -|sigma|, then index"),
    "greedy adds the correction":
        ("            rho = rho - G_rS @ c\n", "            rho = rho + G_rS @ c\n"),
    "greedy uses the wrong Gram rows":
        ("            G_rS = D[rest] @ D[S].T\n", "            G_rS = D[rest] @ D[S[::-1]].T\n"),
    "greedy ties to highest index":
        ("        order = np.lexsort((rest, -a))\n        if rest.size > 1:",
         "        order = np.lexsort((-rest, -a))\n        if rest.size > 1:"),
    "greedy solves on sigma of the pool head":
        ("        c = ridge_coefficients(D[S], sigma[S], ridge_abs, ridge_rel)\n    return S, c, near\n\n\ndef pl_support",
         "        c = ridge_coefficients(D[S], sigma[pool[: len(S)]], ridge_abs, ridge_rel)\n    return S, c, near\n\n\ndef pl_support"),
    "residual adds the reconstruction":
        ("    r = x - (D[list(S)].T @ c if len(S) else 0.0)",
         "    r = x + (D[list(S)].T @ c if len(S) else 0.0)"),
    "trigger at e >= delta":
        ("    flags = FLAG_TRIGGER if e > delta else 0", "    flags = FLAG_TRIGGER if e >= delta else 0"),
    "keys use the value delta":
        ("return self.delta_key if dict_index % 2 == 0 else self.delta_value",
         "return self.delta_value if dict_index % 2 == 0 else self.delta_key"),
    "adapt commits triggering rows too":
        ("    for m in range(idx.shape[0]):\n        if not trig[m]:",
         "    for m in range(idx.shape[0]):\n        if True:"),
    "adapt orders candidates by index only":
        ("cand = sorted(eligible, key=lambda j: (usage[j], j))", "cand = sorted(eligible)"),
    "adapt may take atoms selected this step":
        ("eligible = [j for j in range(N) if usage[j] < p.tau_c and not touched[j]]",
         "eligible = [j for j in range(N) if usage[j] < p.tau_c]"),
    "adapt writes the unnormalised vector":
        ("a = round_to_storage(x / np.sqrt(np.dot(x, x)), dtype)", "a = round_to_storage(x, dtype)"),
    "adapt code without ridge":
        ("c = float(np.dot(a, x)) / ((1.0 + p.ridge_rel) * g + p.ridge_abs)",
         "c = float(np.dot(a, x)) / g"),
    "bf16 rounding truncates":
        ("r = np.ldexp(np.rint(np.ldexp(w, -q)), q)", "r = np.ldexp(np.trunc(np.ldexp(w, -q)), q)"),
    "bf16 keeps one bit too many":
        ("q = np.maximum(e - 8, -133)", "q = np.maximum(e - 9, -133)"),
    "reconstruct skips the first slot":
        ("            for k in range(s):\n                j = idx[t, m, k]",
         "            for k in range(1, s):\n                j = idx[t, m, k]"),
    "append overwrites from slot 0":
        ("    nxt = int(n_atoms)\n", "    nxt = 0\n"),
    "append skips the usage commit":
        ("    trig = (flags & FLAG_TRIGGER) != 0\n    _commit_nontriggering(usage, idx, trig)\n    replaced",
         "    trig = (flags & FLAG_TRIGGER) != 0\n    replaced"),
    "append ignores the capacity":
        ("        if nxt < cap:\n", "        if nxt < cap + 1:\n"),
    "yardstick screens a pool first":
        ("        pool, near_pool = np.arange(D.shape[0]), False\n",
         "        pool, near_pool = candidate_pool(sigma, p.n)\n"),
    "replay bounds the yardstick by the pool size":
        ("    n_eff = N if p.select == \"omp\" else p.n", "    n_eff = p.n"),
    "recall counts empty slots":
        ("            if j >= 0:\n                total += 1", "            if True:\n                total += 1"),
    "recall against the wrong vector's pool":
        ("    for pv, sv in zip(P, S):", "    for pv, sv in zip(P[::-1], S):"),
    "PL takes the pool head unsorted":
        ("    S = [int(j) for j in pool[order[:s]]]", "    S = [int(j) for j in pool[::-1][:s]]"),
    "greedy may re-pick a chosen atom":
        ("        rest = np.array([j for j in pool if j not in S], dtype=np.int64)\n",
         "        rest = np.array(list(pool), dtype=np.int64)\n"),
    "greedy uses least-squares coefficients inside the loop":
        ("        c = ridge_coefficients(D[S], sigma[S], ridge_abs, ridge_rel)\n    return S, c, near\n\n\ndef pl_support",
         "        c = ridge_coefficients(D[S], sigma[S], 0.0, 0.0)\n"
         "    c = ridge_coefficients(D[S], sigma[S], ridge_abs, ridge_rel)\n    return S, c, near\n\n\ndef pl_support"),
    "replay skips the PL check":
        ("            if a[j] < a_s * (1 - TIE_REL):\n", "            if False:\n"),
    "replay checks picks against the sure set, not the given pool":
        ("        candidates = np.array(sorted(Pset), dtype=np.int64)\n",
         "        candidates = sure\n"),
    "replay accepts a pick outside its own pool":
        ("            if j not in Pset:\n", "            if False:\n"),
    "replay accepts a pool without a sure atom":
        ("        if missing:\n", "        if False:\n"),
    "replay accepts a pool of the wrong size":
        ("        if len(Pset) != len(P) or len(P) != n_eff:\n", "        if len(Pset) != len(P):\n"),
}

PIN_TESTS = [f for name, f in sorted(vars(pins).items())
             if name.startswith("test_") and callable(f)]


def _mutated_module(old, new):
    assert SRC.count(old) == 1, f"mutation text matches {SRC.count(old)} times"
    mod = types.ModuleType("oracle_mutant")
    sys.modules["oracle_mutant"] = mod          # dataclasses look their module up by name
    try:
        exec(compile(SRC.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    finally:
        del sys.modules["oracle_mutant"]
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name, monkeypatch):
    old, new = MUTATIONS[name]
    mod = _mutated_module(old, new)
    for attr in dir(ofk):
        if not attr.startswith("__") and hasattr(mod, attr):
            monkeypatch.setattr(oracle, attr, getattr(mod, attr), raising=False)
    monkeypatch.setattr(pins, "_round_bf16", mod._round_bf16)
    monkeypatch.setattr(pins, "OracleParams", mod.OracleParams)
    failed = []
    for f in PIN_TESTS:
        try:
            f()
        except Exception:          # AssertionError or a crash both count as caught
            failed.append(f.__name__)
    assert failed, f"no pin caught mutation {name!r}"


def test_unmutated_copy_passes_every_pin(monkeypatch):
    mod = _mutated_module("TIE_REL = 1e-5", "TIE_REL = 1e-5")
    for attr in dir(ofk):
        if not attr.startswith("__") and hasattr(mod, attr):
            monkeypatch.setattr(oracle, attr, getattr(mod, attr), raising=False)
    for f in PIN_TESTS:
        f()
