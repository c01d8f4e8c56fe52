"""Plain CPU oracle for decode attention over sparse-coded keys and values.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this module.  It shares no code with the HIP library.

Source: the abstract of "FAD-KV: Adaptive Dictionary KV Caching for Efficient Reasoning
Decoding" stores every token's key and value as a sparse combination of dictionary atoms; a
decode step then attends the new query over those stored tokens.  The pages give no formula
for that step, so the oracle takes the plainest one: rebuild each cached key and value from
its code, k_t = sum_k cK[t][k] d^K_{iK[t][k]} (empty slots, idx < 0, contribute nothing), and
apply standard scaled softmax attention,

    out = sum_t p_t v_t,   p = softmax_t(scale * <q, k_t>),   over the row's len tokens,

with out = 0 for a row without tokens.  Everything is float64 from the stored values.
"""
from __future__ import annotations

import numpy as np


def rebuild(D: np.ndarray, idx: np.ndarray, coef: np.ndarray) -> np.ndarray:
    """Rows sum_k coef[t][k] D[idx[t][k]] for a [T][s] code block (idx < 0: empty slot)."""
    D = np.asarray(D, dtype=np.float64)
    T, s = idx.shape
    out = np.zeros((T, D.shape[1]))
    for t in range(T):
        for k in range(s):
            j = int(idx[t, k])
            if 0 <= j < D.shape[0]:
                out[t] += float(coef[t, k]) * D[j]
    return out


def attend_row(Dk, Dv, k_idx, k_coef, v_idx, v_coef, q, scale: float) -> np.ndarray:
    """Attention of the queries q [G][d] over one row's tokens (codes [len][s])."""
    q = np.asarray(q, dtype=np.float64)
    G, d = q.shape
    if k_idx.shape[0] == 0:
        return np.zeros((G, d))
    K = rebuild(Dk, k_idx, k_coef)
    V = rebuild(Dv, v_idx, v_coef)
    out = np.zeros((G, d))
    for g in range(G):
        z = scale * (K @ q[g])
        z = z - z.max()
        p = np.exp(z)
        p = p / p.sum()
        out[g] = p @ V
    return out


def attend(Dk, Dv, k_idx, k_coef, v_idx, v_coef, lens, q, scale: float) -> np.ndarray:
    """out [R][G][d] for codes [R][T][s], lens [R] (tokens t < lens[r] count), q [R][G][d]."""
    R = k_idx.shape[0]
    G, d = q.shape[1], q.shape[2]
    out = np.zeros((R, G, d))
    for r in range(R):
        L = int(lens[r])
        out[r] = attend_row(Dk, Dv, k_idx[r, :L], k_coef[r, :L], v_idx[r, :L], v_coef[r, :L],
                            q[r], scale)
    return out
