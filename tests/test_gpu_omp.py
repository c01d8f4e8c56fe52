"""GPU parity of the full-dictionary greedy yardstick (fadkv_encode_omp, through the C ABI)
and of the pool-recall diagnostic against the CPU oracle (select="omp", pool_recall).

Same comparison rules as the encoder's parity (tests/parity.py): atoms in selection order
bit-exact unless the oracle flags a near-tie (margin <= 1e-5 relative), where the GPU's choice
is validated by replay; coefficients and relative errors within 1e-4 relative.  The
yardstick's correlations are sums of exact products of the stored atoms with the fp32
residual (split into storage-dtype parts), accumulated in fp32, like the encoder's scores.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import OracleParams
from sparse_dictionary_coding_amd import fadkv, synth
from sparse_dictionary_coding_amd.synth import SyntheticKV, Workload, to_f64

from . import parity

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _banner(msg):
    print(f"[gpu-omp] {msg}", flush=True)


def _omp_params(p: fadkv.Params) -> OracleParams:
    return oracle.with_select(parity.oracle_params(p), "omp")


SHAPES = [
    # dtype, d, N, s, M, T, anisotropic
    ("f32", 64, 300, 5, 50, 2, False),
    ("f16", 128, 1000, 8, 77, 2, True),
    ("bf16", 128, 1000, 8, 77, 2, True),
    ("f16", 64, 513, 12, 33, 3, False),
    ("bf16", 64, 640, 6, 65, 1, True),
    ("f32", 128, 256, 4, 31, 2, False),
    ("bf16", 128, 2048, 16, 40, 1, True),
    ("f16", 128, 1024, 32, 20, 1, True),
    ("f16", 64, 100, 1, 40, 1, False),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "-".join(map(str, s[:6])))
def test_omp_parity_shapes(shape):
    dtype, d, N, s, M, T, aniso = shape
    _banner(f"omp {shape}")
    w = Workload("omp", T, 1, d, N, max(s, min(N, 64)), s, dtype, 1, M, min(s, 8), 0.0, 0.2,
                 (3 * d) // 4 if aniso else None, 17 + N)
    g = SyntheticKV(w)
    A = g.atoms()
    X = g.batch(A)
    X[0, 3] = 0                              # zero vector: empty code, error 0
    X[-1, 5, 7] = float("inf")               # non-finite input
    p = fadkv.Params(n=w.n, s=s)
    codes = fadkv.fadkv_encode_omp(A.to(DEV), X.to(DEV), p)
    torch.cuda.synchronize()
    rep, _ = parity.compare_encode(to_f64(A), to_f64(X), parity.codes_to_numpy(codes),
                                   _omp_params(p))
    rep.check()
    assert rep.nonfinite == 1
    assert rep.exact >= 0.8 * rep.vectors


def test_omp_is_deterministic_and_reuses_its_workspace():
    _banner("omp determinism")
    w = Workload("omp", 2, 1, 128, 1500, 64, 8, "bf16", 1, 45, 8, 0.0, 0.2, 96, 5)
    g = SyntheticKV(w, device=DEV)
    A = g.atoms()
    p = fadkv.Params(n=64, s=8)
    ws = torch.empty(fadkv.fadkv_omp_workspace_bytes(A, p, 45), dtype=torch.uint8, device=DEV)
    X1, X2 = g.batch(A, step=0), g.batch(A, step=1)
    a = parity.codes_to_numpy(fadkv.fadkv_encode_omp(A, X1, p, workspace=ws))
    fadkv.fadkv_encode_omp(A, X2, p, workspace=ws)
    b = parity.codes_to_numpy(fadkv.fadkv_encode_omp(A, X1, p, workspace=ws))
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


def test_omp_full_size_llama3b_decode_sampled_and_pool_recall():
    """The 3B decode step (56 dictionaries x 256 vectors, N = 4096 fp16, s = 8) in the launch
    configuration the benchmark times: sampled rows against the oracle's yardstick, and the
    pool recall (share of yardstick atoms inside fadkv_screen's Top-256 pool) per sampled row
    against the oracle's pool and yardstick on the same row."""
    w = synth.WORKLOADS["llama3b_decode"]
    _banner(f"omp full size {w.name}")
    g = SyntheticKV(w, device=DEV)
    A = g.atoms()
    X = g.batch(A)
    p = fadkv.Params(n=w.n, s=w.s)
    codes = fadkv.fadkv_encode_omp(A, X, p)
    pool = fadkv.Pool.empty(w.num_dicts, w.M, w.n, DEV)
    fadkv.fadkv_screen(A, X, p, out=pool)
    torch.cuda.synchronize()
    gi, gc, ge, gf = parity.codes_to_numpy(codes)
    pidx = pool.atom_indices().cpu().numpy()
    op = _omp_params(p)
    rng = np.random.default_rng(8)
    rows = sorted(set(zip(rng.integers(0, w.num_dicts, 40).tolist(),
                          rng.integers(0, w.M, 40).tolist())))
    Af = to_f64(A)
    rep = parity.Report()
    hits_gpu = hits_ref = total = 0
    for (t, m) in rows:
        x = X[t, m].float().cpu().double().numpy()
        delta = op.delta(t)
        oc = oracle.encode_vector(Af[t], x, op, delta)
        parity.compare_vector(rep, f"dict {t} row {m}", Af[t], x, gi[t, m], gc[t, m], ge[t, m],
                              int(gf[t, m]), oc, op, delta)
        ref_pool, near = oracle.candidate_pool(Af[t] @ x, w.n)
        if oc.ties or near:
            continue
        assert set(pidx[t, m].tolist()) == set(ref_pool.tolist())
        hg = oracle.pool_recall(pidx[t, m][None], gi[t, m][None]) * np.sum(gi[t, m] >= 0)
        hr = oracle.pool_recall(ref_pool[None], oc.idx[None]) * np.sum(oc.idx >= 0)
        assert round(hg) == round(hr)
        hits_gpu += round(hg)
        hits_ref += round(hr)
        total += int(np.sum(oc.idx >= 0))
    rep.check()
    assert hits_gpu == hits_ref and total > 0
    _banner(f"  {rep.vectors} rows ({rep.near_tie} near-tie), recall on the sample "
            f"{hits_ref / total:.3f}")
