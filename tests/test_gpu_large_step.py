"""GPU parity of the screening path on prefill-sized steps (thousands of vectors per
dictionary, many workgroups per dictionary).

Every row's candidate pool is compared with the oracle's (exact set wherever the oracle sees
no near-tie at the Top-n boundary, else a valid pool), and the full encode is compared with the
oracle on sampled rows.  Shapes span ragged atom tiles and ragged vector blocks, both head
dims, n up to 512, and inputs whose boundary bins overflow the boundary buffer so that the
refinement sweeps run.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_dictionary_coding_amd import fadkv
from sparse_dictionary_coding_amd.synth import SyntheticKV, Workload, to_f64

from . import parity

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _banner(msg):
    print(f"[gpu-large-step] {msg}", flush=True)


def _pool_check(Af, Xf, pool: fadkv.Pool, n, exact_only=False):
    """Compare every row's pool with the oracle's; returns (rows, near-tie rows)."""
    pidx = pool.idx.cpu().numpy().astype(np.int64) & 0xFFFF
    psig = pool.score.cpu().numpy().astype(np.float64)
    status = pool.status.cpu().numpy()
    T, M = Xf.shape[0], Xf.shape[1]
    near_rows = 0
    for t in range(T):
        S = Xf[t] @ Af[t].T                                  # [M][N] fp64 scores
        for m in range(M):
            x = Xf[t, m]
            if not np.all(np.isfinite(x)):
                assert status[t, m] == 2, (t, m)
                continue
            if not np.any(x):
                assert status[t, m] == 1, (t, m)
                continue
            assert status[t, m] == 0, (t, m)
            sig = S[m]
            P, near = oracle.candidate_pool(sig, n)
            got = pidx[t, m]
            assert len(set(got.tolist())) == n, (t, m, "duplicate pool entries")
            assert np.all(got < Af.shape[1]), (t, m)
            if near and not exact_only:
                near_rows += 1
                a = np.abs(sig)
                thr = np.sort(a)[::-1][n - 1]
                assert np.all(a[got] >= thr * (1 - 1e-5) - 1e-12), (t, m)
                continue
            assert set(got.tolist()) == set(P.tolist()), (t, m)
            assert np.max(np.abs(psig[t, m] - sig[got])) <= 1e-5 * np.max(np.abs(sig[P])) + 1e-6
    return T * M, near_rows


CASES = [
    # dtype, d, N, n, s, M, T, anisotropic atoms
    ("bf16", 128, 1000, 64, 8, 2100, 1, True),      # ragged atom tile, ragged vector block
    ("f16", 64, 3000, 256, 8, 2048, 2, False),      # head_dim 64
    ("f16", 128, 4096, 256, 8, 2080, 1, True),      # 3B dictionary shape
    ("bf16", 128, 8192, 512, 16, 2048, 1, True),    # 8B shape: boundary bins near the buffer size
    ("f32", 64, 700, 32, 4, 2300, 1, False),        # fp32 dictionary (16x16x4 fp32 MFMA path)
    ("bf16", 64, 2500, 128, 8, 2200, 2, True),      # bf16, head_dim 64
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c[:6])))
def test_large_step_screen_and_encode_parity(case):
    dtype, d, N, n, s, M, T, aniso = case
    _banner(f"case {case}")
    w = Workload("large_step", T, 1, d, N, n, s, dtype, 1, M, min(s, 8), 0.05, 0.2,
                 (3 * d) // 4 if aniso else None, 17)
    g = SyntheticKV(w)
    A = g.atoms()
    X = g.batch(A)
    Ad, Xd = A.to(DEV), X.to(DEV)
    p = fadkv.Params(n=n, s=s)
    pool = fadkv.fadkv_screen(Ad, Xd, p)
    torch.cuda.synchronize()
    Af, Xf = to_f64(A), to_f64(X)
    rows, near = _pool_check(Af, Xf, pool, n)
    _banner(f"  pools: {rows} rows, {near} near-tie")
    # the encode through the same kernels, sampled rows against the oracle
    codes = fadkv.fadkv_encode(Ad, Xd, p)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    sample = sorted({(int(t), int(m)) for t, m in zip(rng.integers(0, T, 96), rng.integers(0, M, 96))})
    sample += [(T - 1, M - 1)]                        # the last row of the ragged block
    rep, _ = parity.compare_encode(Af, Xf, parity.codes_to_numpy(codes), parity.oracle_params(p),
                                   rows=sample)
    rep.check()


def test_large_step_edge_cases_and_refinement():
    """Zero and non-finite rows inside a large step; an atom set where each |score| value is
    shared by 128 atoms (boundary bins far over the buffer, so the refinement sweeps decide the
    pool, ties to the lowest index); n = N."""
    _banner("edge cases")
    rng = np.random.default_rng(9)
    d, N, M = 64, 1024, 2048 + 37
    # atom j = +-e_(j % 8): |<atom, x>| = |x_(j % 8)|, every value shared by 128 atoms, exactly
    A = np.zeros((1, N, d))
    j = np.arange(N)
    A[0, j, j % 8] = np.where((j // 8) % 2 == 0, 1.0, -1.0)
    X = rng.standard_normal((1, M, d))
    X[0, 0] = 0.0
    X[0, 5, 3] = np.nan
    X[0, 6, 1] = np.inf
    X[0, M - 1] = 0.0
    X = oracle.round_to_storage(X, "f16")
    At = torch.from_numpy(A).to(torch.float16).to(DEV)
    Xt = torch.from_numpy(X).to(torch.float16).to(DEV)
    for n in (200, 300, 512):
        pool = fadkv.fadkv_screen(At, Xt, fadkv.Params(n=n, s=4))
        torch.cuda.synchronize()
        # scores are exact in fp32, so even the exact ties must resolve as the oracle does
        rows, _ = _pool_check(A, X, pool, n, exact_only=True)
        _banner(f"  duplicated-value atoms, n={n}: {rows} rows")
    # a generic dictionary with a pool of every atom (n = N)
    N2 = 300
    A2 = rng.standard_normal((1, N2, d))
    A2 /= np.linalg.norm(A2, axis=2, keepdims=True)
    A2 = oracle.round_to_storage(A2, "bf16")
    X2 = oracle.round_to_storage(rng.standard_normal((1, 2048, d)), "bf16")
    At2 = torch.from_numpy(A2).to(torch.bfloat16).to(DEV)
    Xt2 = torch.from_numpy(X2).to(torch.bfloat16).to(DEV)
    pool = fadkv.fadkv_screen(At2, Xt2, fadkv.Params(n=N2, s=4))
    torch.cuda.synchronize()
    rows, _ = _pool_check(A2, X2, pool, N2)
    _banner(f"  n = N = {N2}: {rows} rows")
