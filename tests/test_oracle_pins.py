"""Pins of the CPU oracle to things other than itself (closed forms, brute force, textbook
routines, invariants and the pages' tables).  CPU only.

Each test names the oracle function it pins and the kind of mistake it is there to catch.
"""
import itertools
import json
import os

import numpy as np
import pytest
import scipy.linalg

import oracle
from oracle import OracleParams
from oracle.fadkv_oracle import (FLAG_EXHAUSTED, FLAG_NONFINITE, FLAG_REPLACED, FLAG_TRIGGER,
                                 _round_bf16)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def unit_rows(a):
    return a / np.linalg.norm(a, axis=1, keepdims=True)


# ---------------------------------------------------------------------------------------
# storage rounding: brute force over every representable value of the format
# ---------------------------------------------------------------------------------------

def _all_values(bits_to_f64, count):
    vals = bits_to_f64(np.arange(count, dtype=np.uint32))
    fin = np.isfinite(vals)
    pats = np.arange(count, dtype=np.uint32)[fin]
    vals = vals[fin]
    order = np.argsort(vals, kind="stable")
    vals, pats = vals[order], pats[order]
    keep = np.concatenate([[True], np.diff(vals) != 0])   # drop -0 duplicate of +0
    return vals[keep], pats[keep]


def _nearest_even(v, vals, pats):
    i = np.searchsorted(vals, v)
    lo, hi = vals[max(i - 1, 0)], vals[min(i, len(vals) - 1)]
    if v == hi:
        return hi
    dl, dh = v - lo, hi - v
    if dl < dh:
        return lo
    if dh < dl:
        return hi
    plo, phi = pats[max(i - 1, 0)], pats[min(i, len(vals) - 1)]
    return lo if (plo & 1) == 0 else hi


def _probe_values(rng, scale):
    v = rng.standard_normal(3000) * scale
    # exact midpoints between neighbours exercise ties-to-even
    return v


def test_bf16_rounding_is_nearest_even_bruteforce():
    """pins round_to_storage('bf16'): wrong shift, truncation or ties-away fail here."""
    with np.errstate(invalid="ignore"):
        vals, pats = _all_values(
            lambda b: ((b << 16).astype(np.uint32)).view(np.float32).astype(np.float64), 1 << 16)
    rng = np.random.default_rng(1)
    probes = list(_probe_values(rng, 1.0)) + list(_probe_values(rng, 1e-38)) + [
        1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 2.0 ** -133 * 1.5,
        2.0 ** -134, 3.0 * 2.0 ** -134]
    for v in probes:
        assert _round_bf16(np.array([v]))[0] == _nearest_even(v, vals, pats), v


def test_f16_rounding_is_nearest_even_bruteforce():
    """pins round_to_storage('f16') (NumPy's float64 -> float16) against brute force."""
    vals, pats = _all_values(
        lambda b: b.astype(np.uint16).view(np.float16).astype(np.float64), 1 << 16)
    rng = np.random.default_rng(2)
    probes = list(_probe_values(rng, 1.0)) + list(_probe_values(rng, 1e-6)) + [
        1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 2.0 ** -25, 3 * 2.0 ** -26]
    for v in probes:
        assert oracle.round_to_storage(np.array([v]), "f16")[0] == _nearest_even(v, vals, pats)


# ---------------------------------------------------------------------------------------
# a1 screening scores
# ---------------------------------------------------------------------------------------

def test_scores_identity_dictionary_returns_x():
    """pins screening_scores: with D = I the scores are x itself."""
    x = np.random.default_rng(0).standard_normal(16)
    np.testing.assert_array_equal(oracle.screening_scores(np.eye(16), x), x)


def test_scores_match_python_loops():
    """pins screening_scores: a transposed operand or wrong axis fails on a non-square D."""
    rng = np.random.default_rng(3)
    D = rng.standard_normal((7, 5))
    x = rng.standard_normal(5)
    ref = [sum(D[j][i] * x[i] for i in range(5)) for j in range(7)]
    np.testing.assert_allclose(oracle.screening_scores(D, x), ref, rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------------------------------
# a2 pool
# ---------------------------------------------------------------------------------------

def test_pool_matches_python_sort():
    """pins candidate_pool: ranking by |sigma| (not sigma) then lowest index."""
    rng = np.random.default_rng(4)
    for _ in range(50):
        N, n = 40, 9
        sig = np.round(rng.standard_normal(N), 1)   # coarse values -> many exact ties
        P, _ = oracle.candidate_pool(sig, n)
        ref = sorted(range(N), key=lambda j: (-abs(sig[j]), j))[:n]
        assert list(P) == ref


def test_pool_ties_go_to_lowest_index():
    sig = np.array([0.5, -2.0, 1.0, 2.0, -1.0, 1.0])
    P, near = oracle.candidate_pool(sig, 3)
    assert list(P) == [1, 3, 2]
    assert near  # 1.0 (index 2) vs 1.0 (index 4) at the boundary


def test_pool_with_n_equal_N_is_everything():
    sig = np.random.default_rng(5).standard_normal(12)
    P, near = oracle.candidate_pool(sig, 12)
    assert sorted(P) == list(range(12)) and not near


def test_pool_near_tie_flag_threshold():
    sig = np.array([1.0, 0.5, 0.5 * (1 - 0.5e-5), 0.1])
    assert oracle.candidate_pool(sig, 2)[1]
    sig = np.array([1.0, 0.5, 0.5 * (1 - 2e-5), 0.1])
    assert not oracle.candidate_pool(sig, 2)[1]


# ---------------------------------------------------------------------------------------
# a4 ridge
# ---------------------------------------------------------------------------------------

def test_ridge_normal_equations_and_cholesky():
    """pins ridge_coefficients: residual of the normal equations and scipy's cho_solve."""
    rng = np.random.default_rng(6)
    for s in (1, 3, 8, 16):
        D_S = unit_rows(rng.standard_normal((s, 32))) * rng.uniform(0.5, 2, (s, 1))
        b = rng.standard_normal(s)
        c = oracle.ridge_coefficients(D_S, b, 1e-4, 0.2)
        G = D_S @ D_S.T
        A = G + np.diag(1e-4 + 0.2 * np.diag(G))
        assert np.linalg.norm(A @ c - b) <= 1e-12 * np.linalg.norm(b)
        np.testing.assert_allclose(c, scipy.linalg.cho_solve(scipy.linalg.cho_factor(A), b),
                                   rtol=1e-11, atol=1e-13)


def test_ridge_system_diagonal_is_1p2_G_plus_1em4():
    """pins ridge_system against Table 5's lambda with non-unit diagonal (catches abs/rel swaps
    and a lambda that ignores diag(G))."""
    G = np.array([[4.0, 1.0], [1.0, 9.0]])
    A = oracle.ridge_system(G, 1e-4, 0.2)
    np.testing.assert_allclose(A, np.array([[4.8001, 1.0], [1.0, 10.8001]]), rtol=1e-15, atol=0)


# ---------------------------------------------------------------------------------------
# a3 GM / PL
# ---------------------------------------------------------------------------------------

def test_gm_s1_closed_form():
    """s = 1: S = argmax|sigma| and c = sigma_j / (1.2 G_jj + 1e-4), with non-unit atoms."""
    rng = np.random.default_rng(7)
    D = unit_rows(rng.standard_normal((30, 12))) * rng.uniform(0.5, 3.0, (30, 1))
    x = rng.standard_normal(12)
    p = OracleParams(n=10, s=1)
    vc = oracle.encode_vector(D, x, p, 0.5)
    sig = D @ x
    j = int(np.argmax(np.abs(sig)))
    assert vc.idx[0] == j
    g = D[j] @ D[j]
    assert vc.coef[0] == pytest.approx(sig[j] / (1.2 * g + 1e-4), rel=1e-13)
    e = np.linalg.norm(x - vc.coef[0] * D[j]) / np.linalg.norm(x)
    assert vc.relerr == pytest.approx(e, rel=1e-13)


def test_gm_ties_go_to_lowest_index():
    """Two identical atoms (indices 1 and 3) tie exactly at the first greedy step: the lower
    index is taken, and its duplicate is then passed over for the next-best atom."""
    D = np.array([[0.0, 1, 0], [1, 0, 0], [0, 0, 1], [1, 0, 0]])
    x = np.array([1.0, 0.5, 0.0])
    gm = oracle.encode_vector(D, x, OracleParams(n=4, s=2), 0.5)
    assert list(gm.idx) == [1, 0]      # rho_3 = 1 - 1/1.2001 < rho_0 = 0.5
    assert gm.ties & oracle.fadkv_oracle.TIE_GREEDY
    # PL ranks by |sigma| alone: both duplicates, lower index first
    pl = oracle.encode_vector(D, x, OracleParams(n=4, s=2, select="pl"), 0.5)
    assert list(pl.idx) == [1, 3]


def test_gm_never_repicks_a_chosen_atom_by_hand():
    """D = I (4 atoms), x = 3 e0 + 0.1 e1, s = 2.  Step 1 takes atom 0 with c0 = 3/1.2001.
    At step 2 the chosen atom still correlates with the residual, rho_0 = 3 (1 - 1/1.2001)
    = 0.50021, more than rho_1 = 0.1: a greedy that does not exclude chosen atoms takes atom 0
    again.  Excluding it gives S = [0, 1], c = (3, 0.1)/1.2001 (G = I, so the ridge system is
    diagonal)."""
    D = np.eye(4)
    x = np.array([3.0, 0.1, 0.0, 0.0])
    vc = oracle.encode_vector(D, x, OracleParams(n=4, s=2), 0.5)
    assert list(vc.idx) == [0, 1]
    np.testing.assert_allclose(vc.coef, [3.0 / 1.2001, 0.1 / 1.2001], rtol=1e-13)
    assert vc.ties == 0


def test_gm_rho_uses_the_ridge_coefficients_by_hand():
    """Three unit atoms d0 = e0, d1 = 0.9 e0 + sqrt(0.19) e1, d2 = e2 and x = (1, x1, 0.1) with
    x1 = 0.05 / sqrt(0.19), so sigma = (1, 0.95, 0.1) and G_10 = 0.9, G_20 = 0.

    Step 1 takes atom 0.  With the Table 5 ridge inside the greedy, c0 = 1/1.2001 and
    rho_1 = 0.95 - 0.9/1.2001 = 0.20006 beats rho_2 = 0.1: S = [0, 1].  A greedy that uses
    least-squares coefficients during the steps (c0 = 1) would see rho_1 = 0.05 < 0.1 and take
    atom 2.  The final coefficients solve the 2x2 system [[1.2001, 0.9], [0.9, 1.2001]] c =
    (1, 0.95), written out by Cramer's rule."""
    r = np.sqrt(0.19)
    D = np.array([[1.0, 0.0, 0.0], [0.9, r, 0.0], [0.0, 0.0, 1.0]])
    x = np.array([1.0, 0.05 / r, 0.1])
    vc = oracle.encode_vector(D, x, OracleParams(n=3, s=2), 0.5)
    assert list(vc.idx) == [0, 1]
    a, b, det = 1.2001, 0.9, 1.2001 ** 2 - 0.81
    c_ref = [(a * 1.0 - b * 0.95) / det, (a * 0.95 - b * 1.0) / det]
    np.testing.assert_allclose(vc.coef, c_ref, rtol=1e-12)
    resid = x - c_ref[0] * D[0] - c_ref[1] * D[1]
    assert vc.relerr == pytest.approx(np.linalg.norm(resid) / np.linalg.norm(x), rel=1e-12)


def test_gm_orthonormal_closed_form():
    """Orthonormal D (G = I): S = the s largest |sigma| in order, c = sigma_S / 1.2001 and
    e^2 = (||x||^2 - ||sigma_S||^2 + (0.2001/1.2001)^2 ||sigma_S||^2) / ||x||^2."""
    rng = np.random.default_rng(8)
    d = 24
    Q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    for s, n in ((4, 10), (6, 24), (3, 3)):
        x = rng.standard_normal(d)
        vc = oracle.encode_vector(Q, x, OracleParams(n=n, s=s), 0.5)
        sig = Q @ x
        ref = list(np.argsort(-np.abs(sig), kind="stable")[:s])
        assert list(vc.idx) == ref
        np.testing.assert_allclose(vc.coef, sig[ref] / 1.2001, rtol=1e-12)
        ss = np.sum(sig[ref] ** 2)
        e2 = (x @ x - ss + (0.2001 / 1.2001) ** 2 * ss) / (x @ x)
        assert vc.relerr == pytest.approx(np.sqrt(e2), rel=1e-12)


def test_gm_with_full_pool_and_no_ridge_is_textbook_omp():
    """n = N and lambda = 0 reduce GM to OMP: supports (as sets) and least-squares coefficients
    match scikit-learn's orthogonal_mp.  Catches sign or index mistakes in the rho update."""
    from sklearn.linear_model import orthogonal_mp
    rng = np.random.default_rng(9)
    checked = 0
    for trial in range(40):
        N, d, s = 60, 20, 5
        D = unit_rows(rng.standard_normal((N, d)))
        x = rng.standard_normal(d)
        p = OracleParams(n=N, s=s, ridge_abs=0.0, ridge_rel=0.0)
        vc = oracle.encode_vector(D, x, p, 0.5)
        if vc.ties:
            continue
        ref = orthogonal_mp(D.T, x, n_nonzero_coefs=s)
        assert set(np.flatnonzero(ref)) == set(vc.idx.tolist())
        np.testing.assert_allclose(ref[vc.idx], vc.coef, rtol=1e-8, atol=1e-10)
        checked += 1
    assert checked >= 30


def _low_coherence_dictionary():
    H = scipy.linalg.hadamard(16) / 4.0
    return np.vstack([np.eye(16), H])      # 32 unit atoms, mutual coherence 1/4


def test_gm_exact_recovery_and_best_subset_low_coherence():
    """Mutual coherence 1/4 < 1/(2s-1) for s = 2: greedy pursuit must recover every planted
    2-sparse vector, and brute force over all C(32,2) subsets finds the same unique
    zero-error support (lambda = 0, n = N)."""
    D = _low_coherence_dictionary()
    N = D.shape[0]
    rng = np.random.default_rng(10)
    p = OracleParams(n=N, s=2, ridge_abs=0.0, ridge_rel=0.0)
    for _ in range(60):
        S = rng.choice(N, 2, replace=False)
        a = rng.uniform(0.5, 2.0, 2) * rng.choice([-1, 1], 2)
        x = a @ D[S]
        vc = oracle.encode_vector(D, x, p, 0.5)
        assert set(vc.idx.tolist()) == set(S.tolist())
        assert vc.relerr < 1e-12
        best = min(itertools.combinations(range(N), 2),
                   key=lambda T: np.linalg.norm(
                       x - D[list(T)].T @ np.linalg.lstsq(D[list(T)].T, x, rcond=None)[0]))
        assert set(best) == set(S.tolist())


def test_gm_best_subset_on_tiny_random_dictionaries():
    """Brute force best-s-subset (N = 24, d = 16, s <= 3) on planted noise-free vectors with
    |a| in [0.5, 2]: the planted support is the unique zero-error subset; where GM (full pool,
    lambda = 0) reaches zero error its support must be that subset."""
    rng = np.random.default_rng(11)
    agree = total = 0
    for trial in range(30):
        s = 1 + trial % 3
        D = unit_rows(rng.standard_normal((24, 16)))
        S = rng.choice(24, s, replace=False)
        a = rng.uniform(0.5, 2.0, s) * rng.choice([-1, 1], s)
        x = a @ D[S]
        errs = {}
        for T in itertools.combinations(range(24), s):
            DT = D[list(T)].T
            r = x - DT @ np.linalg.lstsq(DT, x, rcond=None)[0]
            errs[T] = np.linalg.norm(r) / np.linalg.norm(x)
        best = min(errs, key=errs.get)
        assert set(best) == set(S.tolist()) and errs[best] < 1e-12
        vc = oracle.encode_vector(D, x, OracleParams(n=24, s=s, ridge_abs=0.0, ridge_rel=0.0), 0.5)
        if vc.relerr < 1e-10:
            assert set(vc.idx.tolist()) == set(S.tolist())
            agree += 1
        total += 1
    assert agree >= total // 2


def test_gm_planted_recovery_tiny_workload_shape():
    """Tiny-workload shape (N=256, d=64, s=4), noise-free planted vectors with |a_i| in
    [0.3, 1.3]: with the whole dictionary as pool the greedy recovers every planted support,
    and at n = 32 it recovers every vector whose planted atoms all made the pool (a missed
    recovery then can only come from the screening, not from the greedy or the ridge)."""
    rng = np.random.default_rng(12)
    D = unit_rows(rng.standard_normal((256, 64)))
    in_pool = 0
    for _ in range(200):
        S = rng.choice(256, 4, replace=False)
        a = rng.uniform(0.3, 1.3, 4) * rng.choice([-1, 1], 4)
        x = a @ D[S]
        full = oracle.encode_vector(D, x, OracleParams(n=256, s=4), 0.5)
        assert set(full.idx.tolist()) == set(S.tolist())
        P, _ = oracle.candidate_pool(D @ x, 32)
        if set(S.tolist()) <= set(P.tolist()):
            vc = oracle.encode_vector(D, x, OracleParams(n=32, s=4), 0.5)
            assert set(vc.idx.tolist()) == set(S.tolist())
            in_pool += 1
    assert in_pool >= 120


def test_pl_takes_the_s_largest_of_the_pool():
    rng = np.random.default_rng(13)
    D = unit_rows(rng.standard_normal((50, 10)))
    x = rng.standard_normal(10)
    p = OracleParams(n=20, s=5, select="pl")
    vc = oracle.encode_vector(D, x, p, 0.5)
    sig = D @ x
    ref = sorted(range(50), key=lambda j: (-abs(sig[j]), j))[:5]
    assert list(vc.idx) == ref
    np.testing.assert_allclose(vc.coef, oracle.ridge_coefficients(D[ref], sig[ref], 1e-4, 0.2),
                               rtol=1e-13)


def test_pl_equals_gm_on_orthonormal_dictionary():
    rng = np.random.default_rng(14)
    Q, _ = np.linalg.qr(rng.standard_normal((16, 16)))
    x = rng.standard_normal(16)
    a = oracle.encode_vector(Q, x, OracleParams(n=8, s=4, select="pl"), 0.5)
    b = oracle.encode_vector(Q, x, OracleParams(n=8, s=4, select="gm"), 0.5)
    assert list(a.idx) == list(b.idx)
    np.testing.assert_allclose(a.coef, b.coef, rtol=1e-12)


# ---------------------------------------------------------------------------------------
# a5 residual, reconstruct, special inputs
# ---------------------------------------------------------------------------------------

def test_relerr_agrees_with_reconstruct():
    rng = np.random.default_rng(15)
    D = unit_rows(rng.standard_normal((64, 16)))
    X = rng.standard_normal((1, 20, 16))
    p = OracleParams(n=16, s=3)
    codes = oracle.encode(D[None], X, p)
    xh = oracle.reconstruct(D[None], codes.idx, codes.coef)
    e = np.linalg.norm(X - xh, axis=2) / np.linalg.norm(X, axis=2)
    np.testing.assert_allclose(codes.relerr, e, rtol=1e-12)


def test_reconstruct_by_hand():
    D = np.arange(12, dtype=np.float64).reshape(1, 4, 3)
    idx = np.array([[[2, 0, -1]]], dtype=np.int32)
    coef = np.array([[[0.5, -1.0, 7.0]]])
    np.testing.assert_array_equal(oracle.reconstruct(D, idx, coef)[0, 0],
                                  0.5 * np.array([6, 7, 8.0]) - np.array([0, 1, 2.0]))


def test_zero_and_nonfinite_vectors():
    D = unit_rows(np.random.default_rng(16).standard_normal((20, 8)))
    p = OracleParams(n=5, s=2)
    z = oracle.encode_vector(D, np.zeros(8), p, 0.5)
    assert list(z.idx) == [-1, -1] and z.relerr == 0.0 and z.flags == 0
    x = np.ones(8)
    x[3] = np.nan
    nf = oracle.encode_vector(D, x, p, 0.5)
    assert list(nf.idx) == [-1, -1] and np.isnan(nf.relerr) and nf.flags == FLAG_NONFINITE


def test_delta_by_dictionary_parity_and_strict_threshold():
    """Keys (even dictionaries) use 0.50, values (odd) 0.70; trigger is e > delta."""
    p = OracleParams()
    assert p.delta(0) == 0.5 and p.delta(1) == 0.7 and p.delta(54) == 0.5 and p.delta(55) == 0.7
    Q = np.eye(4)
    x = np.array([1.0, 0.0, 0.0, 0.0])
    # one atom equal to x: e = 0.2001/1.2001 exactly representable check of strictness
    vc = oracle.encode_vector(Q, x, OracleParams(n=2, s=1), 0.2001 / 1.2001)
    assert not (vc.flags & FLAG_TRIGGER)


# ---------------------------------------------------------------------------------------
# a6 adaptation invariants
# ---------------------------------------------------------------------------------------

def _adapt_run(steps=8, rows=64, tau_c=1, seed=20, N=256, d=64, s=4, n=32, drift=0.2,
               support_limit=192):
    rng = np.random.default_rng(seed)
    atoms = oracle.round_to_storage(unit_rows(rng.standard_normal((1, N, d))[0]), "f32")[None]
    usage = np.zeros((1, N), dtype=np.int64)
    p = OracleParams(n=n, s=s, tau_c=tau_c)
    history = []
    for step in range(steps):
        X = np.empty((1, rows, d))
        for m in range(rows):
            if rng.uniform() < drift:
                X[0, m] = rng.standard_normal(d)
            else:
                S = rng.choice(support_limit, s, replace=False)
                X[0, m] = rng.standard_normal(s) @ atoms[0, S]
        X = oracle.round_to_storage(X, "f32")
        codes = oracle.encode(atoms, X, p)
        new_atoms, new_usage, new_codes, replaced = oracle.adapt(atoms, usage, X, codes, p, "f32")
        history.append((atoms, usage, X, codes, new_atoms, new_usage, new_codes, replaced))
        atoms, usage = new_atoms, new_usage
    return p, history


def test_adapt_keeps_size_and_counts_usage():
    p, hist = _adapt_run()
    committed = 0
    replaced_total = 0
    for atoms, usage, X, codes, na, nu, nc, rep in hist:
        assert na.shape == atoms.shape and nu.shape == usage.shape   # N never changes
        committed += int(np.sum(nc.idx >= 0))
        assert int(nu.sum()) == committed                             # sum usage = slots
        replaced_total += int(np.sum(rep >= 0))
    assert replaced_total > 0


def test_adapt_replaced_atom_and_code():
    p, hist = _adapt_run()
    seen = 0
    for atoms, usage, X, codes, na, nu, nc, rep in hist:
        for m in np.flatnonzero(rep[0] >= 0):
            j = rep[0, m]
            x = X[0, m]
            a = oracle.round_to_storage(x / np.linalg.norm(x), "f32")
            np.testing.assert_array_equal(na[0, j], a)
            assert nu[0, j] == 1 and usage[0, j] < p.tau_c
            assert nc.idx[0, m, 0] == j and np.all(nc.idx[0, m, 1:] == -1)
            g = a @ a
            assert nc.coef[0, m, 0] == pytest.approx((a @ x) / (1.2 * g + 1e-4), rel=1e-13)
            assert nc.relerr[0, m] == pytest.approx(0.2001 / 1.2001, rel=1e-5)
            assert nc.flags[0, m] & FLAG_REPLACED and nc.flags[0, m] & FLAG_TRIGGER
            seen += 1
    assert seen > 0


def test_adapt_never_overwrites_a_referenced_atom():
    """With tau_c = 1 no committed code of any step references an atom overwritten later."""
    p, hist = _adapt_run(steps=10)
    live = set()   # atoms referenced by committed codes so far
    for atoms, usage, X, codes, na, nu, nc, rep in hist:
        step_sel = set(int(j) for j in codes.idx[0].ravel() if j >= 0)
        for j in rep[0][rep[0] >= 0]:
            assert int(j) not in live and int(j) not in step_sel
        live |= set(int(j) for j in nc.idx[0].ravel() if j >= 0)
        # untouched atoms keep their values bit for bit
        mask = np.ones(atoms.shape[1], bool)
        mask[rep[0][rep[0] >= 0]] = False
        np.testing.assert_array_equal(atoms[0, mask], na[0, mask])


def test_adapt_swapping_two_triggering_rows_swaps_their_slots():
    """Slots are handed out in row order: after swapping two triggering rows, each vector
    lands in the other's slot, so the two written atoms trade contents and nothing else moves."""
    p, hist = _adapt_run(steps=1)
    atoms, usage, X, codes, na, nu, nc, rep = hist[0]
    trig = np.flatnonzero(codes.flags[0] & FLAG_TRIGGER)
    assert trig.size >= 2
    a, b = trig[0], trig[-1]
    ja, jb = rep[0, a], rep[0, b]
    assert ja >= 0 and jb >= 0 and ja != jb
    perm = np.arange(X.shape[1])
    perm[a], perm[b] = b, a
    codes2 = oracle.Codes(codes.idx[:, perm], codes.coef[:, perm], codes.relerr[:, perm],
                          codes.flags[:, perm], codes.ties[:, perm])
    na2, nu2, _, rep2 = oracle.adapt(atoms, usage, X[:, perm], codes2, p, "f32")
    np.testing.assert_array_equal(rep2, rep)
    np.testing.assert_array_equal(na2[0, ja], na[0, jb])
    np.testing.assert_array_equal(na2[0, jb], na[0, ja])
    rest = np.ones(atoms.shape[1], bool)
    rest[[ja, jb]] = False
    np.testing.assert_array_equal(na2[0, rest], na[0, rest])
    np.testing.assert_array_equal(nu2, nu)


def test_adapt_candidates_ordered_by_usage_then_index():
    """tau_c = 3, preset usage: candidates are taken in (usage, index) order, skipping atoms
    with usage >= tau_c and atoms selected by this step's codes."""
    N, d = 8, 4
    A = np.vstack([np.eye(4), -np.eye(4)])[None]
    usage = np.array([[2, 0, 5, 1, 0, 2, 1, 3]])
    X = np.ones((1, 4, d))
    X[0, :, 0] = [1, 2, 3, 4]
    idx = np.full((1, 4, 1), -1, np.int32)
    idx[0, 2, 0] = 4          # a triggering row whose code uses atom 4 protects it
    codes = oracle.Codes(idx, np.zeros((1, 4, 1)), np.ones((1, 4)),
                         np.full((1, 4), FLAG_TRIGGER, np.uint8), np.zeros((1, 4), np.uint8))
    p = OracleParams(n=1, s=1, tau_c=3)
    _, nu, nc, rep = oracle.adapt(A, usage, X, codes, p, "f32")
    # eligible: usage<3 and not atom 4 -> {1:0, 3:1, 6:1, 0:2, 5:2}; order 1,3,6,0 for 4 rows
    assert list(rep[0]) == [1, 3, 6, 0]


def test_adapt_exhaustion_when_no_inactive_atom():
    p, hist = _adapt_run(steps=1)
    atoms, usage, X, codes, *_ = hist[0]
    full = np.full_like(usage, p.tau_c)
    na, nu, nc, rep = oracle.adapt(atoms, full, X, codes, p, "f32")
    trig = (codes.flags[0] & FLAG_TRIGGER) != 0
    assert trig.any()
    assert np.all(rep == -1)
    assert np.all((nc.flags[0][trig] & FLAG_EXHAUSTED) != 0)
    np.testing.assert_array_equal(na, atoms)
    assert int(nu.sum() - full.sum()) == int(np.sum(codes.idx >= 0))


def test_adapt_delta_extremes():
    rng = np.random.default_rng(21)
    D = unit_rows(rng.standard_normal((1, 64, 16)))
    X = rng.standard_normal((1, 10, 16))
    X[0, 3] = 0.0
    lo = oracle.encode(D, X, OracleParams(n=8, s=2, delta_key=0.0))
    hi = oracle.encode(D, X, OracleParams(n=8, s=2, delta_key=np.inf))
    assert (lo.flags[0] & FLAG_TRIGGER).sum() == 9          # every non-zero row
    assert (hi.flags[0] & FLAG_TRIGGER).sum() == 0
    # an infinite delta is never near: the trigger decision there is not a near-tie
    assert not np.any(hi.ties & oracle.fadkv_oracle.TIE_DELTA)


# ---------------------------------------------------------------------------------------
# append-only growth (the abstract's contrast; Fig. 3a)
# ---------------------------------------------------------------------------------------

def _append_run(steps=4, rows=64, cap_extra=400, seed=22, N=128, d=32, s=4, n=32, drift=0.25):
    rng = np.random.default_rng(seed)
    cap = N + cap_extra
    atoms = np.zeros((1, cap, d))
    atoms[0, :N] = oracle.round_to_storage(unit_rows(rng.standard_normal((N, d))), "f32")
    usage = np.zeros((1, cap), dtype=np.int64)
    n_atoms = np.array([N])
    p = OracleParams(n=n, s=s)
    hist = []
    for step in range(steps):
        X = np.empty((1, rows, d))
        for m in range(rows):
            if rng.uniform() < drift:
                X[0, m] = rng.standard_normal(d)
            else:
                S = rng.choice(N, s, replace=False)
                X[0, m] = rng.standard_normal(s) @ atoms[0, S]
        X = oracle.round_to_storage(X, "f32")
        codes = oracle.encode(atoms, X, p)
        out = oracle.append(atoms, usage, X, codes, n_atoms, p, "f32")
        hist.append((atoms, usage, n_atoms, X, codes) + out)
        atoms, usage, _, _, n_atoms = out
    return p, hist


def test_append_grows_by_one_atom_per_trigger_in_row_order():
    p, hist = _append_run()
    committed = 0
    for atoms, usage, n0, X, codes, na, nu, nc, rep, n1 in hist:
        trig = np.flatnonzero(codes.flags[0] & FLAG_TRIGGER)
        assert trig.size > 0
        assert int(n1[0]) == int(n0[0]) + trig.size
        assert list(rep[0][trig]) == list(range(int(n0[0]), int(n1[0])))
        for m in trig:
            x = X[0, m]
            np.testing.assert_array_equal(na[0, rep[0, m]], oracle.round_to_storage(x / np.linalg.norm(x), "f32"))
            assert nu[0, rep[0, m]] == 1 and nc.idx[0, m, 0] == rep[0, m]
        np.testing.assert_array_equal(na[0, :int(n0[0])], atoms[0, :int(n0[0])])   # never overwrites
        assert np.all(na[0, int(n1[0]):] == 0.0)
        committed += int(np.sum(nc.idx >= 0))
        assert int(nu.sum()) == committed


def test_append_stops_at_capacity():
    p, hist = _append_run(steps=1)
    atoms, usage, n0, X, codes, *_ = hist[0]
    trig = np.flatnonzero(codes.flags[0] & FLAG_TRIGGER)
    assert trig.size > 2
    small = atoms[:, : int(n0[0]) + 2]
    na, nu, nc, rep, n1 = oracle.append(small, usage[:, : small.shape[1]], X, codes, n0, p, "f32")
    assert int(n1[0]) == small.shape[1]
    assert list(np.flatnonzero(rep[0] >= 0)) == list(trig[:2])
    assert np.all(nc.flags[0][trig[2:]] & FLAG_EXHAUSTED)


def test_append_and_replace_code_the_trigger_alike():
    """The same step committed both ways: every triggering row gets the same one-atom code
    (coefficient and error) whether its atom is appended or overwrites an inactive one."""
    p, hist = _append_run(steps=1)
    atoms, usage, n0, X, codes, na, nu, nc, rep, n1 = hist[0]
    fa, fu, fc, frep = oracle.adapt(atoms, usage, X, codes, p, "f32")
    trig = np.flatnonzero(codes.flags[0] & FLAG_TRIGGER)
    assert np.all(frep[0][trig] >= 0)
    np.testing.assert_array_equal(fc.coef[0, trig], nc.coef[0, trig])
    np.testing.assert_array_equal(fc.relerr[0, trig], nc.relerr[0, trig])


def test_zero_padding_is_never_selected():
    p, hist = _append_run(steps=1)
    atoms, usage, n0, X, codes, *_ = hist[0]
    tight = oracle.encode(atoms[:, : int(n0[0])], X, p)
    np.testing.assert_array_equal(tight.idx, codes.idx)
    np.testing.assert_array_equal(tight.coef, codes.coef)


# ---------------------------------------------------------------------------------------
# the pages' tables
# ---------------------------------------------------------------------------------------

def test_cost_model_reproduces_table4_cost_column():
    """Reading of GM/PL: screening costs N*d MACs per vector, GM's greedy s*n*d, PL's solve
    s*s*d; against full OMP (s*N*d) this gives Table 4's 0.19 and 0.13 at N=4096, s=8, n=256."""
    g = json.load(open(os.path.join(GOLDEN, "table4_efficiency.json")))
    N, s, n = g["model_shape"]["N"], g["model_shape"]["s"], g["model_shape"]["n"]
    gm = (N + s * n) / (s * N)
    pl = (N + s * s) / (s * N)
    assert round(gm, 2) == g["rows"]["GM (ours)"][0] == g["rows"]["FAD-KV (GM)"][0]
    assert round(pl, 2) == g["rows"]["PL (ours)"][0]
    for name, row in g["rows"].items():
        assert row[2] == pytest.approx(1000.0 / row[1], abs=0.01)     # tok/s = 1000 / ms
        if row[3] is not None:
            assert row[3] == pytest.approx(53.63 / row[1] - 1, abs=0.0006)


def test_table5_defaults():
    g = json.load(open(os.path.join(GOLDEN, "table5_hyperparameters.json")))
    p = OracleParams()
    assert (p.n, p.s) == (g["by_model_size"]["3B"]["n"], g["by_model_size"]["3B"]["s"])
    assert p.ridge_abs == g["ridge"]["abs"] and p.ridge_rel == g["ridge"]["rel_diag_G"]
    assert p.delta_key == g["delta"]["key"] and p.delta_value == g["delta"]["value"]


# ---------------------------------------------------------------------------------------
# full-dictionary yardstick ("omp") and the pool-recall diagnostic (Fig. 1b)
# ---------------------------------------------------------------------------------------

def test_omp_is_textbook_omp_whatever_the_pool_size():
    """select="omp" with lambda = 0 is OMP over the whole dictionary even when n is far below
    N: supports (as sets) and least-squares coefficients match scikit-learn's orthogonal_mp.
    Catches a yardstick that screens a pool first."""
    from sklearn.linear_model import orthogonal_mp
    rng = np.random.default_rng(31)
    checked = outside = 0
    for trial in range(40):
        N, d, s = 60, 20, 5
        D = unit_rows(rng.standard_normal((N, d)))
        x = rng.standard_normal(d)
        p = OracleParams(n=s, s=s, ridge_abs=0.0, ridge_rel=0.0, select="omp")
        vc = oracle.encode_vector(D, x, p, 0.5)
        if vc.ties:
            continue
        ref = orthogonal_mp(D.T, x, n_nonzero_coefs=s)
        assert set(np.flatnonzero(ref)) == set(vc.idx.tolist())
        np.testing.assert_allclose(ref[vc.idx], vc.coef, rtol=1e-8, atol=1e-10)
        top = set(np.argsort(-np.abs(D @ x))[:s].tolist())
        outside += int(not set(vc.idx.tolist()) <= top)
        checked += 1
    assert checked >= 30 and outside >= 5


def test_gm_equals_omp_when_the_pool_holds_every_omp_pick():
    """If each full-dictionary greedy pick lies in the Top-n pool, GM (same ridge) makes the
    same picks in the same order with the same coefficients; vectors where an OMP atom is
    missing from the pool are where the two may part (and some must, at this pool size)."""
    rng = np.random.default_rng(32)
    N, d, s, n = 200, 32, 6, 40
    D = unit_rows(rng.standard_normal((N, d)))
    same = differ = 0
    for _ in range(120):
        x = rng.standard_normal(d)
        po = OracleParams(n=n, s=s, select="omp")
        pg = OracleParams(n=n, s=s, select="gm")
        vo = oracle.encode_vector(D, x, po, 0.5)
        vg = oracle.encode_vector(D, x, pg, 0.5)
        if vo.ties or vg.ties:
            continue
        pool, _ = oracle.candidate_pool(D @ x, n)
        if set(vo.idx.tolist()) <= set(pool.tolist()):
            assert vo.idx.tolist() == vg.idx.tolist()
            np.testing.assert_allclose(vo.coef, vg.coef, rtol=1e-12)
            assert vo.relerr == pytest.approx(vg.relerr, rel=1e-12)
            same += 1
        else:
            differ += 1
            assert vo.relerr <= vg.relerr * (1 + 1e-9) or vo.idx.tolist() != vg.idx.tolist()
    assert same >= 10 and differ >= 5


def test_replay_accepts_own_choices_and_rejects_a_swapped_atom():
    """replay_support validates a support chosen elsewhere: the oracle's own GM, PL and
    yardstick supports pass, and replacing one atom by the atom of smallest |score| fails."""
    rng = np.random.default_rng(33)
    N, d, s, n = 80, 16, 4, 8
    D = unit_rows(rng.standard_normal((N, d)))
    for sel in ("gm", "pl", "omp"):
        p = OracleParams(n=n, s=s, select=sel)
        ok = 0
        for _ in range(20):
            x = rng.standard_normal(d)
            vc = oracle.encode_vector(D, x, p, 0.5)
            valid, why, c, e = oracle.replay_support(D, x, vc.idx, p)
            assert valid, (sel, why)
            np.testing.assert_allclose(c, vc.coef, rtol=1e-10)
            worst = int(np.argmin(np.abs(D @ x)))
            if worst in vc.idx:
                continue
            bad = vc.idx.copy()
            bad[-1] = worst
            assert not oracle.replay_support(D, x, bad, p)[0], sel
            ok += 1
        assert ok >= 15


def test_replay_pl_rejects_an_atom_outside_the_s_largest():
    """D = I (8 atoms), x = (8, 7, ..., 1), n = 6, s = 3: PL must take {0, 1, 2}.  Atom 4 is in
    every valid pool (|sigma| = 4 is the 5th largest) but not among the 3 largest, so a PL
    support [0, 1, 4] is invalid; [2, 0, 1] (same set, any order) is valid."""
    D = np.eye(8)
    x = np.arange(8.0, 0.0, -1.0)
    p = OracleParams(n=6, s=3, select="pl")
    assert oracle.replay_support(D, x, [2, 0, 1], p)[0]
    valid, why, _, _ = oracle.replay_support(D, x, [0, 1, 4], p)
    assert not valid and "s largest" in why
    assert not oracle.replay_support(D, x, [0, 1, 4], p, pool=[0, 1, 2, 3, 4, 5])[0]


def _tie_at_pool_boundary():
    """d0 = e0, d1 = e1, d2 = 0.6 e0 + 0.8 e2, d3 = e3 and x = (5, 1, -5, 2): sigma =
    (5, 1, -1, 2) up to rounding of 0.6 and 0.8, so with n = 3 atoms 1 and 2 tie for the third
    pool place (sure set {0, 3}).  GM takes atom 0 first (c0 = 5/1.2001); then
    rho_1 = 1, rho_2 = -1 - 0.6 c0 = -3.4998, rho_3 = 2."""
    D = np.array([[1.0, 0, 0, 0], [0, 1.0, 0, 0], [0.6, 0, 0.8, 0], [0, 0, 0, 1.0]])
    x = np.array([5.0, 1.0, -5.0, 2.0])
    return D, x


def test_replay_with_the_coder_pool():
    """replay_support against the pool the coder screened.  With the tie above, pool {0, 2, 3}
    is valid; inside it GM must take atom 2 at step 2 (|rho| 3.4998).  A coder that took
    atom 3 (|rho| 2) passed over a better atom of its own pool: only the pool-aware check sees
    that, since atom 2 is not in the sure set.  Pool {0, 1, 3} is valid too, and then [0, 3]
    is right (atom 2 is not in that pool, rho_3 = 2 > rho_1 = 1); [0, 1] is a pick from
    outside the pool {0, 2, 3}; a pool that leaves out the sure atom 3 or has the wrong size is
    invalid."""
    D, x = _tie_at_pool_boundary()
    p = OracleParams(n=3, s=2)
    sig = D @ x
    assert abs(abs(sig[1]) - abs(sig[2])) <= 1e-12
    assert oracle.replay_support(D, x, [0, 2], p, pool=[0, 2, 3])[0]
    assert oracle.replay_support(D, x, [0, 3], p)[0]            # blind to the pool
    valid, why, _, _ = oracle.replay_support(D, x, [0, 3], p, pool=[0, 2, 3])
    assert not valid and "below best" in why
    assert oracle.replay_support(D, x, [0, 3], p, pool=[0, 1, 3])[0]
    valid, why, _, _ = oracle.replay_support(D, x, [0, 1], p, pool=[0, 2, 3])
    assert not valid and "own pool" in why
    assert not oracle.replay_support(D, x, [0, 2], p, pool=[0, 1, 2])[0]
    assert not oracle.replay_support(D, x, [0, 2], p, pool=[0, 2, 3, 1])[0]
    # PL inside the coder's pool: the two largest |sigma| of {0, 1, 3} are atoms 0 and 3
    pl = OracleParams(n=3, s=2, select="pl")
    assert oracle.replay_support(D, x, [0, 3], pl, pool=[0, 1, 3])[0]
    assert not oracle.replay_support(D, x, [0, 1], pl, pool=[0, 1, 3])[0]


def test_pool_recall_by_hand():
    pool = np.array([[3, 1, 7], [0, 2, 4]])
    supp = np.array([[1, 7, 9, -1], [4, -1, -1, -1]])
    assert oracle.pool_recall(pool, supp) == pytest.approx(3 / 4)
    assert oracle.pool_recall(pool, -np.ones((2, 4), int)) == 1.0
    assert oracle.pool_recall(pool[None], supp[None]) == pytest.approx(3 / 4)


def test_pool_recall_is_one_on_planted_incoherent_vectors():
    """Mutual coherence 1/4, planted 2-sparse vectors with coefficients +-1: a planted atom
    scores at least 1 - 1/4 and any other at most 2/4, so the yardstick recovers the support
    and the pool of the 2 largest |scores| is exactly it: recall 1.  A pool of 1 holds one of
    the two atoms: recall 1/2."""
    D = _low_coherence_dictionary()
    rng = np.random.default_rng(34)
    pools, pools1, supps = [], [], []
    p = OracleParams(n=4, s=2, ridge_abs=0.0, ridge_rel=0.0, select="omp")
    for _ in range(40):
        S = rng.choice(D.shape[0], 2, replace=False)
        a = rng.choice([-1.0, 1.0], 2)
        x = a @ D[S]
        vc = oracle.encode_vector(D, x, p, 0.5)
        assert set(vc.idx.tolist()) == set(S.tolist())
        pools.append(oracle.candidate_pool(D @ x, 2)[0])
        pools1.append(oracle.candidate_pool(D @ x, 1)[0])
        supps.append(vc.idx)
    assert oracle.pool_recall(np.array(pools), np.array(supps)) == 1.0
    assert oracle.pool_recall(np.array(pools1), np.array(supps)) == 0.5
