"""Plain CPU oracle for FAD-KV's screening sparse coder and fixed-size dictionary adaptation.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this module.  It shares no code, table or helper with the HIP
library in ``sparse_dictionary_coding_amd/`` and never imports it; inputs reach it as NumPy
arrays holding the exact stored values (atoms and vectors already in their storage dtype).

Sources (arXiv 2610.37921, "FAD-KV: Adaptive Dictionary KV Caching for Efficient Reasoning
Decoding", as shown on its summary pages):
  * Abstract: every key/value vector is stored as a sparse combination of dictionary atoms;
    the coder screens the whole dictionary once, keeps a Top-n candidate pool and then refines
    coefficients cheaply; adaptation reuses inactive atoms so the dictionary never grows.
  * Figure 1 caption: scores are dictionary correlations; the Top-n pool recalls the atoms a
    full OMP would pick; many atoms stay unused after prefill.
  * Figure 2 caption: when a vector's reconstruction error is high, an inactive atom is
    overwritten by a context-relevant atom instead of appending one; N is constant.
  * Table 4: "GM" and "FAD-KV (GM)" coding cost 0.19 of full OMP, "PL" 0.13.
  * Table 5: N, s, n per model size; ridge 1e-4 + 0.20 diag(G); delta 0.50 key / 0.70 value.

Everything is computed in float64 from the stored values.  Where the pages leave a step
open, the reading taken is stated at the function that implements it:
  * GM = greedy pursuit restricted to the pool (orthogonal-matching style, with the Table 5
    ridge system solved at every step); PL = the s largest |score| of the pool, one solve.
    The yardstick "omp" (Fig. 1b's full-OMP atoms, Table 4's Cost 1.00) is the same greedy
    with every atom a candidate, so it differs from GM only by the screening.
    (Table 4's cost column: (N + s*n)/(s*N) = 0.1875 and (N + s*s)/(s*N) = 0.127.)
  * scores are raw inner products <d_j, x>, ranked by absolute value; every tie goes to the
    lowest atom index;
  * the error is the relative l2 residual ||x - D_S^T c|| / ||x|| and triggers when > delta;
  * an atom is inactive at commit when its usage counter is below tau_c and no vector of the
    step selected it; the new atom is x/||x|| rounded to the storage dtype, and the triggering
    vector is re-coded onto that single atom with the one-atom ridge coefficient.

Decisions that floating point takes (pool boundary, greedy argmax, error vs delta) are marked
``near-tie`` when their margin is at most 1e-5 relative: a kernel in fp32 may legitimately
decide those the other way, so parity checks validate them instead of comparing them.

Parity pins for every function live in tests/test_oracle_pins.py.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional, Sequence

import numpy as np

# Per-vector flag bits (shared meaning with the C-ABI's flags byte; values restated there).
FLAG_TRIGGER = 0x01    # relative error above delta
FLAG_REPLACED = 0x02   # adaptation overwrote an inactive atom with this vector's direction
FLAG_EXHAUSTED = 0x04  # triggered, but no inactive atom was left this step
FLAG_NONFINITE = 0x08  # input held a NaN or Inf: empty code, error NaN
FLAG_NEAR_TIE = 0x10   # oracle only: some decision had a margin <= TIE_REL

# Which decision was a near-tie (diagnostic detail of FLAG_NEAR_TIE).
TIE_POOL = 0x1      # |score| at the pool boundary
TIE_GREEDY = 0x2    # greedy argmax (or PL's s-th place inside the pool)
TIE_DELTA = 0x4     # relative error vs delta

TIE_REL = 1e-5

DTYPES = ("f32", "f16", "bf16")


@dataclass(frozen=True)
class OracleParams:
    """Hyperparameters of one encode/adapt call (defaults: Table 5, 3B/4B column)."""

    n: int = 256                 # candidate-pool size
    s: int = 8                   # sparsity budget
    ridge_abs: float = 1e-4      # lambda = ridge_abs + ridge_rel * diag(G)
    ridge_rel: float = 0.20
    delta_key: float = 0.50      # even dictionaries hold keys
    delta_value: float = 0.70    # odd dictionaries hold values
    tau_c: int = 1               # inactive <=> usage < tau_c
    select: str = "gm"           # "gm" greedy in pool, "pl" s largest of pool, "omp" greedy
                                 # over the whole dictionary (the yardstick; n unused)

    def delta(self, dict_index: int) -> float:
        return self.delta_key if dict_index % 2 == 0 else self.delta_value


# ----------------------------------------------------------------------------------------
# Storage rounding (round-to-nearest, ties-to-even, straight from float64)
# ----------------------------------------------------------------------------------------

_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def _round_bf16(v: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 value (8 significant bits, binary32 exponent range), ties to even."""
    v = np.asarray(v, dtype=np.float64)
    out = v.copy()
    fin = np.isfinite(v) & (v != 0.0)
    if np.any(fin):
        w = v[fin]
        _, e = np.frexp(w)                       # |w| in [2^(e-1), 2^e)
        q = np.maximum(e - 8, -133)              # spacing 2^(e-8); subnormal spacing 2^-133
        r = np.ldexp(np.rint(np.ldexp(w, -q)), q)  # rint: half to even
        r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, w), r)
        out[fin] = r
    return out


def round_to_storage(v, dtype: str) -> np.ndarray:
    """Round float64 values to the storage dtype and return them as float64."""
    v = np.asarray(v, dtype=np.float64)
    if dtype == "f32":
        return v.astype(np.float32).astype(np.float64)
    if dtype == "f16":
        return v.astype(np.float16).astype(np.float64)
    if dtype == "bf16":
        return _round_bf16(v)
    raise ValueError(f"unknown dtype {dtype!r}")


# ----------------------------------------------------------------------------------------
# a1  screening scores
# ----------------------------------------------------------------------------------------

def screening_scores(D: np.ndarray, x: np.ndarray) -> np.ndarray:
    """sigma_j = <d_j, x> for every atom (Fig. 1: dictionary correlations; atoms unit-norm)."""
    return D @ x


# ----------------------------------------------------------------------------------------
# a2  Top-n candidate pool
# ----------------------------------------------------------------------------------------

def candidate_pool(sigma: np.ndarray, n: int):
    """The n atoms of largest |sigma|, ties to the lowest index (abstract: one-shot Top-n).

    Returns (pool indices in rank order, near_tie) where near_tie says the n-th and (n+1)-th
    |sigma| differ by at most TIE_REL relative.
    """
    N = sigma.shape[0]
    a = np.abs(sigma)
    order = np.lexsort((np.arange(N), -a))   # primary key -|sigma|, then index
    pool = order[:n]
    near = False
    if n < N:
        an, an1 = a[order[n - 1]], a[order[n]]
        near = bool(an - an1 <= TIE_REL * an)
    return pool, near


# ----------------------------------------------------------------------------------------
# a4  Gram + ridge
# ----------------------------------------------------------------------------------------

def ridge_system(G_SS: np.ndarray, ridge_abs: float, ridge_rel: float) -> np.ndarray:
    """G_SS + diag(ridge_abs + ridge_rel * G_jj)  (Table 5: lambda = 1e-4 + 0.20 diag(G))."""
    return G_SS + np.diag(ridge_abs + ridge_rel * np.diag(G_SS))


def ridge_coefficients(D_S: np.ndarray, b: np.ndarray, ridge_abs: float, ridge_rel: float):
    """Solve (G_SS + Lambda_S) c = b with G_SS = D_S D_S^T (the abstract's coefficient step)."""
    G = D_S @ D_S.T
    return np.linalg.solve(ridge_system(G, ridge_abs, ridge_rel), b)


# ----------------------------------------------------------------------------------------
# a3  support inside the pool
# ----------------------------------------------------------------------------------------

def gm_support(D: np.ndarray, sigma: np.ndarray, pool: Sequence[int], s: int,
               ridge_abs: float, ridge_rel: float):
    """GM: s greedy steps inside the pool (Tables 1-4 "GM"; the pages do not expand it).

    Step k: rho_j = sigma_j - sum_{m in S} G_jm c_m for every pool atom not yet chosen, pick
    the largest |rho_j| (ties to the lowest atom index), append it to S and re-solve the ridge
    system on S.  Returns (S in selection order, c, near_tie).
    """
    pool = np.asarray(pool, dtype=np.int64)
    S: list[int] = []
    c = np.zeros(0)
    near = False
    for _ in range(s):
        rest = np.array([j for j in pool if j not in S], dtype=np.int64)
        rho = sigma[rest].copy()
        if S:
            G_rS = D[rest] @ D[S].T
            rho = rho - G_rS @ c
        a = np.abs(rho)
        order = np.lexsort((rest, -a))
        if rest.size > 1:
            b1, b2 = a[order[0]], a[order[1]]
            near = near or bool(b1 - b2 <= TIE_REL * b1)
        S.append(int(rest[order[0]]))
        c = ridge_coefficients(D[S], sigma[S], ridge_abs, ridge_rel)
    return S, c, near


def pl_support(D: np.ndarray, sigma: np.ndarray, pool: Sequence[int], s: int,
               ridge_abs: float, ridge_rel: float):
    """PL: the s pool atoms of largest |sigma| (ties to lowest index), then one ridge solve."""
    pool = np.asarray(pool, dtype=np.int64)
    a = np.abs(sigma[pool])
    order = np.lexsort((pool, -a))
    S = [int(j) for j in pool[order[:s]]]
    near = False
    if s < pool.size:
        near = bool(a[order[s - 1]] - a[order[s]] <= TIE_REL * a[order[s - 1]])
    c = ridge_coefficients(D[S], sigma[S], ridge_abs, ridge_rel)
    return S, c, near


# ----------------------------------------------------------------------------------------
# a5  residual and delta
# ----------------------------------------------------------------------------------------

def relative_residual(D: np.ndarray, x: np.ndarray, S: Sequence[int], c: np.ndarray) -> float:
    """||x - D_S^T c|| / ||x||  (Fig. 2: adaptation fires when this is high)."""
    nx = np.linalg.norm(x)
    if nx == 0.0:
        return 0.0
    r = x - (D[list(S)].T @ c if len(S) else 0.0)
    return float(np.linalg.norm(r) / nx)


# ----------------------------------------------------------------------------------------
# encode: a1..a5 for one vector and for whole dictionaries
# ----------------------------------------------------------------------------------------

@dataclass
class VectorCode:
    idx: np.ndarray        # int32 [s], -1 = empty slot, selection order
    coef: np.ndarray       # float64 [s]
    relerr: float
    flags: int
    ties: int = 0          # TIE_* bits
    pool: Optional[np.ndarray] = None


def encode_vector(D: np.ndarray, x: np.ndarray, p: OracleParams, delta: float) -> VectorCode:
    s = p.s
    idx = np.full(s, -1, dtype=np.int32)
    coef = np.zeros(s)
    if not np.all(np.isfinite(x)):
        return VectorCode(idx, coef, float("nan"), FLAG_NONFINITE)
    if not np.any(x != 0.0):
        # the zero vector is represented exactly by the empty code
        return VectorCode(idx, coef, 0.0, 0)
    sigma = screening_scores(D, x)
    if p.select == "omp":
        # Full-dictionary yardstick (Fig. 1b's "full-OMP atoms", Table 4's Cost = 1.00): the
        # same greedy steps as GM with every atom a candidate, so the only difference from GM
        # is the screening.  There is no pool, hence no pool boundary to be near.
        pool, near_pool = np.arange(D.shape[0]), False
    else:
        pool, near_pool = candidate_pool(sigma, p.n)
    if p.select in ("gm", "omp"):
        S, c, near_sel = gm_support(D, sigma, pool, s, p.ridge_abs, p.ridge_rel)
    elif p.select == "pl":
        S, c, near_sel = pl_support(D, sigma, pool, s, p.ridge_abs, p.ridge_rel)
    else:
        raise ValueError(p.select)
    e = relative_residual(D, x, S, c)
    idx[: len(S)] = S
    coef[: len(S)] = c
    flags = FLAG_TRIGGER if e > delta else 0
    ties = (TIE_POOL if near_pool else 0) | (TIE_GREEDY if near_sel else 0)
    if np.isfinite(delta) and abs(e - delta) <= TIE_REL * delta:
        ties |= TIE_DELTA      # an infinite delta is never approached: no near-tie there
    if ties:
        flags |= FLAG_NEAR_TIE
    return VectorCode(idx, coef, e, flags, ties, pool)


@dataclass
class Codes:
    idx: np.ndarray        # int32 [num_dicts][M][s]
    coef: np.ndarray       # float64 [num_dicts][M][s]
    relerr: np.ndarray     # float64 [num_dicts][M]
    flags: np.ndarray      # uint8 [num_dicts][M]
    ties: np.ndarray       # uint8 [num_dicts][M]

    def copy(self) -> "Codes":
        return Codes(self.idx.copy(), self.coef.copy(), self.relerr.copy(),
                     self.flags.copy(), self.ties.copy())


def encode(atoms: np.ndarray, X: np.ndarray, p: OracleParams,
           dict_ids: Optional[Sequence[int]] = None) -> Codes:
    """Encode X[t][m] against atoms[t] for every dictionary t (rows independent).

    ``dict_ids`` gives each slice's dictionary number when a subset of dictionaries is passed
    (it fixes key/value delta by parity); default 0..num_dicts-1.
    """
    atoms = np.asarray(atoms, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64)
    T, M = X.shape[0], X.shape[1]
    ids = list(range(T)) if dict_ids is None else list(dict_ids)
    out = Codes(np.full((T, M, p.s), -1, np.int32), np.zeros((T, M, p.s)),
                np.zeros((T, M)), np.zeros((T, M), np.uint8), np.zeros((T, M), np.uint8))
    for t in range(T):
        delta = p.delta(ids[t])
        for m in range(M):
            vc = encode_vector(atoms[t], X[t, m], p, delta)
            out.idx[t, m] = vc.idx
            out.coef[t, m] = vc.coef
            out.relerr[t, m] = vc.relerr
            out.flags[t, m] = vc.flags
            out.ties[t, m] = vc.ties
    return out


# ----------------------------------------------------------------------------------------
# a6  fixed-size adaptation
# ----------------------------------------------------------------------------------------

def _commit_nontriggering(usage: np.ndarray, idx: np.ndarray, trig: np.ndarray):
    """usage[j] += 1 for each atom of each non-triggering code (row order)."""
    for m in range(idx.shape[0]):
        if not trig[m]:
            for j in idx[m]:
                if j >= 0:
                    usage[j] += 1


def _recode_onto_new_atom(A, usage, j, x, idx_m, coef_m, p: OracleParams, dtype: str) -> float:
    """Write the new atom round(x/||x||) into slot j (usage 1) and re-code the row onto it with
    the one-atom ridge coefficient <d_j,x>/((1+rel) G_jj + abs); returns the new error."""
    a = round_to_storage(x / np.sqrt(np.dot(x, x)), dtype)
    A[j] = a
    usage[j] = 1
    g = float(np.dot(a, a))
    c = float(np.dot(a, x)) / ((1.0 + p.ridge_rel) * g + p.ridge_abs)
    idx_m[:] = -1
    coef_m[:] = 0.0
    idx_m[0] = j
    coef_m[0] = c
    return float(np.linalg.norm(x - c * a) / np.linalg.norm(x))


def adapt_dictionary(A: np.ndarray, usage: np.ndarray, X: np.ndarray, idx: np.ndarray,
                     coef: np.ndarray, relerr: np.ndarray, flags: np.ndarray,
                     p: OracleParams, dtype: str):
    """Commit one step of codes for one dictionary, overwriting inactive atoms in place.

    Fig. 2: a badly coded vector replaces an inactive atom rather than growing N.  Every
    vector of the step was encoded against the dictionary as it stood at step start; the
    commit then runs in row order:
      1. usage[j] += 1 for each atom of each non-triggering code;
      2. candidates = atoms with usage < tau_c that no code of this step selected, ordered by
         (usage, index);
      3. the k-th triggering row takes the k-th candidate j: atom j <- round(x/||x||),
         usage[j] <- 1, the row's code becomes ({j}, <d_j,x>/((1+rel) G_jj + abs));
      4. triggering rows beyond the candidates keep their code, commit its usage and are
         flagged exhausted.
    Arrays are modified in place; returns replaced[M] (atom index or -1).
    """
    N = A.shape[0]
    M = X.shape[0]
    trig = (flags & FLAG_TRIGGER) != 0
    touched = np.zeros(N, dtype=bool)
    for m in range(M):
        for j in idx[m]:
            if j >= 0:
                touched[j] = True
    _commit_nontriggering(usage, idx, trig)
    eligible = [j for j in range(N) if usage[j] < p.tau_c and not touched[j]]
    cand = sorted(eligible, key=lambda j: (usage[j], j))
    replaced = np.full(M, -1, dtype=np.int32)
    k = 0
    for m in range(M):
        if not trig[m]:
            continue
        if k < len(cand):
            j = cand[k]
            k += 1
            relerr[m] = _recode_onto_new_atom(A, usage, j, X[m], idx[m], coef[m], p, dtype)
            flags[m] |= FLAG_REPLACED
            replaced[m] = j
        else:
            flags[m] |= FLAG_EXHAUSTED
            for j in idx[m]:
                if j >= 0:
                    usage[j] += 1
    return replaced


def adapt(atoms: np.ndarray, usage: np.ndarray, X: np.ndarray, codes: Codes,
          p: OracleParams, dtype: str):
    """adapt_dictionary over every dictionary; returns (atoms', usage', codes', replaced)."""
    atoms = np.array(atoms, dtype=np.float64, copy=True)
    usage = np.array(usage, dtype=np.int64, copy=True)
    X = np.asarray(X, dtype=np.float64)
    codes = codes.copy()
    T, M = X.shape[0], X.shape[1]
    replaced = np.full((T, M), -1, dtype=np.int32)
    for t in range(T):
        replaced[t] = adapt_dictionary(atoms[t], usage[t], X[t], codes.idx[t], codes.coef[t],
                                       codes.relerr[t], codes.flags[t], p, dtype)
    return atoms, usage, codes, replaced


# ----------------------------------------------------------------------------------------
# append-only growth (the contrast the abstract and Fig. 3a draw)
# ----------------------------------------------------------------------------------------

def append_dictionary(A: np.ndarray, usage: np.ndarray, X: np.ndarray, idx: np.ndarray,
                      coef: np.ndarray, relerr: np.ndarray, flags: np.ndarray, n_atoms: int,
                      p: OracleParams, dtype: str):
    """Commit one step by appending instead of reusing: the abstract contrasts FAD-KV with
    adaptation that only appends atoms, whose dictionary keeps growing during generation
    (Fig. 3a).

    The dictionary is stored with capacity A.shape[0]; its first n_atoms rows are in use and
    the rest are zero (a zero atom scores 0 and is never selected).  Non-triggering rows commit
    usage as in adapt_dictionary; the k-th triggering row (row order) appends round(x/||x||) at
    slot n_atoms + k while the capacity lasts and is re-coded onto it exactly as a replacement
    would be; rows past the capacity keep their code, commit its usage and are flagged
    exhausted.  Arrays are modified in place; returns (replaced[M], new n_atoms).
    """
    cap = A.shape[0]
    M = X.shape[0]
    trig = (flags & FLAG_TRIGGER) != 0
    _commit_nontriggering(usage, idx, trig)
    replaced = np.full(M, -1, dtype=np.int32)
    nxt = int(n_atoms)
    for m in range(M):
        if not trig[m]:
            continue
        if nxt < cap:
            j = nxt
            nxt += 1
            relerr[m] = _recode_onto_new_atom(A, usage, j, X[m], idx[m], coef[m], p, dtype)
            flags[m] |= FLAG_REPLACED
            replaced[m] = j
        else:
            flags[m] |= FLAG_EXHAUSTED
            for j in idx[m]:
                if j >= 0:
                    usage[j] += 1
    return replaced, nxt


def append(atoms: np.ndarray, usage: np.ndarray, X: np.ndarray, codes: Codes,
           n_atoms: np.ndarray, p: OracleParams, dtype: str):
    """append_dictionary over every dictionary; returns (atoms', usage', codes', replaced,
    n_atoms')."""
    atoms = np.array(atoms, dtype=np.float64, copy=True)
    usage = np.array(usage, dtype=np.int64, copy=True)
    X = np.asarray(X, dtype=np.float64)
    codes = codes.copy()
    n_atoms = np.array(n_atoms, dtype=np.int64, copy=True)
    T, M = X.shape[0], X.shape[1]
    replaced = np.full((T, M), -1, dtype=np.int32)
    for t in range(T):
        replaced[t], n_atoms[t] = append_dictionary(atoms[t], usage[t], X[t], codes.idx[t],
                                                    codes.coef[t], codes.relerr[t],
                                                    codes.flags[t], int(n_atoms[t]), p, dtype)
    return atoms, usage, codes, replaced, n_atoms


# ----------------------------------------------------------------------------------------
# reconstruct (boundary call)
# ----------------------------------------------------------------------------------------

def reconstruct(atoms: np.ndarray, idx: np.ndarray, coef: np.ndarray) -> np.ndarray:
    """x_hat = sum_k c_k d_{idx_k} over non-empty slots, per dictionary and row."""
    atoms = np.asarray(atoms, dtype=np.float64)
    T, M, s = idx.shape
    d = atoms.shape[2]
    out = np.zeros((T, M, d))
    for t in range(T):
        for m in range(M):
            for k in range(s):
                j = idx[t, m, k]
                if j >= 0:
                    out[t, m] += coef[t, m, k] * atoms[t, j]
    return out


# ----------------------------------------------------------------------------------------
# validation of a coder's choices at near-ties (used by parity tests)
# ----------------------------------------------------------------------------------------

def replay_support(D: np.ndarray, x: np.ndarray, S_given: Sequence[int], p: OracleParams,
                   pool: Optional[Sequence[int]] = None):
    """Check that a support chosen by another implementation is a valid answer.

    With a_n the n-th largest |sigma|, every valid pool holds the sure set
    {j : |sigma_j| > a_n (1 + TIE_REL)} and nothing outside the possible set
    {j : |sigma_j| >= a_n (1 - TIE_REL)}.  Each given atom must be possible.

    Without ``pool``: for GM each given choice must reach (1 - TIE_REL) times the best |rho|
    over the not-yet-chosen sure atoms at that step; for PL each given atom must reach
    (1 - TIE_REL) times the s-th largest |sigma|.

    With ``pool`` (the candidate pool the other implementation screened, n distinct atoms): the
    pool must itself be a valid Top-n (n distinct possible atoms holding every sure atom), every
    given atom must belong to it, and the choices are checked against that pool: for GM each
    choice must reach (1 - TIE_REL) times the best |rho| over the pool atoms not yet chosen,
    for PL each atom must reach (1 - TIE_REL) times the s-th largest |sigma| of the pool.  A
    greedy that passed over a better atom of its own pool fails here even when that atom is
    not in the sure set.

    Returns (valid, reason, c, e) with c and e computed on the given support.
    """
    S_given = [int(j) for j in S_given if j >= 0]
    sigma = screening_scores(D, x)
    N = sigma.shape[0]
    a = np.abs(sigma)
    order = np.lexsort((np.arange(N), -a))
    n_eff = N if p.select == "omp" else p.n      # the yardstick's "pool" is every atom
    an = a[order[n_eff - 1]]
    possible = set(int(j) for j in range(N) if a[j] >= an * (1 - TIE_REL))
    sure = np.array([j for j in range(N) if a[j] > an * (1 + TIE_REL)], dtype=np.int64)
    for j in S_given:
        if j not in possible:
            return False, f"atom {j} outside every valid pool", None, None
    if len(set(S_given)) != len(S_given):
        return False, "repeated atom", None, None
    if pool is not None:
        P = [int(j) for j in pool]
        Pset = set(P)
        if len(Pset) != len(P) or len(P) != n_eff:
            return False, f"pool of {len(P)} entries ({len(Pset)} distinct), not {n_eff}", None, None
        outside = [j for j in P if j not in possible]
        if outside:
            return False, f"pool atom {outside[0]} outside every valid pool", None, None
        missing = [int(j) for j in sure if int(j) not in Pset]
        if missing:
            return False, f"pool misses the sure atom {missing[0]}", None, None
        for j in S_given:
            if j not in Pset:
                return False, f"atom {j} not in its own pool", None, None
        candidates = np.array(sorted(Pset), dtype=np.int64)
    else:
        candidates = sure
    if p.select == "pl":
        if pool is not None:
            a_s = np.sort(a[candidates])[::-1][p.s - 1]
        else:
            a_s = a[order[p.s - 1]]
        for j in S_given:
            if a[j] < a_s * (1 - TIE_REL):
                return False, f"atom {j} not among the s largest", None, None
    else:
        S: list[int] = []
        c = np.zeros(0)
        for j in S_given:
            rest = np.array([i for i in candidates if i not in S], dtype=np.int64)
            best = 0.0
            if rest.size:
                rho = sigma[rest].copy()
                if S:
                    rho = rho - (D[rest] @ D[S].T) @ c
                best = float(np.max(np.abs(rho)))
            rj = abs(sigma[j] - (float((D[j] @ D[S].T) @ c) if S else 0.0))
            if rj < best * (1 - TIE_REL):
                return False, f"atom {j}: |rho|={rj} below best {best}", None, None
            S.append(j)
            c = ridge_coefficients(D[S], sigma[S], p.ridge_abs, p.ridge_rel)
    c = ridge_coefficients(D[S_given], sigma[S_given], p.ridge_abs, p.ridge_rel)
    e = relative_residual(D, x, S_given, c)
    return True, "", c, e


# ----------------------------------------------------------------------------------------
# pool-recall diagnostic (Fig. 1b)
# ----------------------------------------------------------------------------------------

def pool_recall(pool: np.ndarray, support: np.ndarray) -> float:
    """Share of the full-dictionary atoms that the Top-n pools hold (Fig. 1b: the screened
    pool recalls most full-OMP atoms): sum over vectors of |S_v & P_v| / sum of |S_v|, with
    pool [..., n] and support [..., s] index arrays over the same vectors; support slots
    below 0 are empty and not counted.  Returns 1.0 when no vector has an atom."""
    P = np.asarray(pool).reshape(-1, np.asarray(pool).shape[-1])
    S = np.asarray(support).reshape(-1, np.asarray(support).shape[-1])
    hit = total = 0
    for pv, sv in zip(P, S):
        members = set(int(j) for j in pv)
        for j in sv:
            if j >= 0:
                total += 1
                hit += int(int(j) in members)
    return hit / total if total else 1.0


def with_select(p: OracleParams, select: str) -> OracleParams:
    return replace(p, select=select)
