"""GPU parity of decode attention over sparse-coded K/V (fadkv_attend, through the C ABI)
against the CPU attention oracle.

Codes are seeded and synthetic (random atoms per slot, some empty slots, N(0,1) coefficients);
queries and dictionaries are stored in the dictionary dtype and fed to the oracle as those exact
values.  Tolerance: the kernels compute q . D_K^T with fp32 accumulation of exact 16-bit
products, logits as s-term fp32 sums, exp with a relative error of a few ulp, and value
weights accumulated exactly as 64-bit fixed point from fp32 products (in fp32 atomics, any
order, when N is too large for that), over up to T*s terms, then a d-wide fp32 dot
with D_V over N atoms.  Each stage contributes O(1e-6) relative error for these sizes, so
|out - ref| <= 2e-4 * max|ref| per (row, query) plus 1e-6 leaves a wide margin while any
indexing, scaling or normalisation mistake shows up at O(1).
"""
import numpy as np
import pytest
import torch

from oracle import attend_oracle
from sparse_dictionary_coding_amd import fadkv

pytestmark = pytest.mark.gpu

DEV = "cuda"
TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _banner(msg):
    print(f"[gpu-attend] {msg}", flush=True)


def _case(dtype, d, N, s, R, T, G, layers=2, empty_frac=0.1, seed=0, lens=None):
    g = torch.Generator().manual_seed(seed)
    atoms = torch.randn(2 * layers, N, d, generator=g)
    atoms = (atoms / atoms.norm(dim=2, keepdim=True)).to(TORCH[dtype])
    def codes():
        idx = torch.randint(0, N, (R, T, s), generator=g, dtype=torch.int32)
        idx[torch.rand(R, T, s, generator=g) < empty_frac] = -1
        coef = torch.randn(R, T, s, generator=g)
        return idx, coef
    ki, kc = codes()
    vi, vc = codes()
    q = (torch.randn(R, G, d, generator=g) * 2.0).to(TORCH[dtype])
    if lens is None:
        lens = torch.randint(0, T + 1, (R,), generator=g, dtype=torch.int32)
        lens[0] = T
    return atoms, ki, kc, vi, vc, torch.as_tensor(lens, dtype=torch.int32), q


def _check(atoms, layer, ki, kc, vi, vc, lens, q, scale, rows=None):
    out = fadkv.fadkv_attend(atoms.to(DEV), layer, ki.to(DEV), kc.to(DEV), vi.to(DEV), vc.to(DEV),
                             lens.to(DEV), q.to(DEV), scale)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    A = atoms.double().numpy()
    Dk, Dv = A[2 * layer], A[2 * layer + 1]
    rows = range(ki.shape[0]) if rows is None else rows
    for r in rows:
        L = int(lens[r])
        ref = attend_oracle.attend_row(Dk, Dv, ki[r, :L].numpy(), kc[r, :L].numpy(),
                                       vi[r, :L].numpy(), vc[r, :L].numpy(),
                                       q[r].double().numpy(), scale)
        for g in range(q.shape[1]):
            tol = 2e-4 * np.max(np.abs(ref[g])) + 1e-6
            err = np.max(np.abs(out[r, g] - ref[g]))
            assert err <= tol, (r, g, L, err, tol)
    return out


SHAPES = [
    # dtype, d, N, s, R, T, G
    ("f16", 128, 4096, 8, 12, 300, 3),
    ("bf16", 128, 4096, 8, 10, 257, 4),
    ("f32", 64, 256, 4, 9, 100, 2),
    ("f16", 64, 1000, 5, 7, 33, 1),
    ("bf16", 128, 8192, 16, 5, 120, 4),
    ("f32", 128, 777, 3, 6, 64, 5),
    ("bf16", 64, 16384, 8, 3, 50, 2),      # largest N: fp32 weight accumulation in LDS
]


@pytest.mark.parametrize("dtype,d,N,s,R,T,G", SHAPES)
def test_attend_parity(dtype, d, N, s, R, T, G):
    _banner(f"attend {dtype} d={d} N={N} s={s} R={R} T={T} G={G}")
    case = _case(dtype, d, N, s, R, T, G, seed=N + T)
    _check(*case[:1], 1, *case[1:], scale=1.0 / np.sqrt(d))


def test_attend_edge_cases():
    _banner("attend edge cases")
    # every row empty: out = 0
    atoms, ki, kc, vi, vc, lens, q = _case("f16", 128, 512, 4, 4, 16, 2, lens=[0, 0, 0, 0])
    out = _check(atoms, 0, ki, kc, vi, vc, lens, q, 0.1)
    assert np.all(out == 0.0)
    # one token per row, and a row whose slots are all empty (uniform weights, zero values)
    atoms, ki, kc, vi, vc, lens, q = _case("bf16", 64, 300, 3, 3, 1, 3, lens=[1, 1, 1])
    ki[2], vi[2] = -1, -1
    _check(atoms, 0, ki, kc, vi, vc, lens, q, 0.125)
    # large logits (max shift) and a large G group split over several workgroups
    atoms, ki, kc, vi, vc, lens, q = _case("f32", 128, 4096, 8, 2, 64, 20, lens=[64, 37])
    _check(atoms, 0, ki, kc, vi, vc, lens, q, 4.0)
    # lens beyond T are clamped to T, negative to 0
    atoms, ki, kc, vi, vc, lens, q = _case("f16", 128, 256, 2, 3, 10, 1, lens=[10, 0, 10])
    out_ref = _check(atoms, 0, ki, kc, vi, vc, lens, q, 0.2)
    out = fadkv.fadkv_attend(atoms.to(DEV), 0, ki.to(DEV), kc.to(DEV), vi.to(DEV), vc.to(DEV),
                             torch.tensor([99, -5, 10], dtype=torch.int32, device=DEV),
                             q.to(DEV), 0.2).cpu().numpy()
    np.testing.assert_allclose(out, out_ref, rtol=1e-5, atol=1e-6)


def test_attend_decode_shape_sampled():
    """The 3B decode shape of one layer (8 KV heads x 32 sequences, 3 query heads each, N = 4096,
    s = 8) with 2048 cached tokens per row; the oracle checks a seeded sample of rows."""
    _banner("attend 3B decode layer, 2048 tokens, sampled rows")
    atoms, ki, kc, vi, vc, lens, q = _case("f16", 128, 4096, 8, 256, 2048, 3, layers=1,
                                           empty_frac=0.02, seed=11)
    rows = np.random.default_rng(3).choice(256, 6, replace=False)
    _check(atoms, 0, ki, kc, vi, vc, lens, q, 1.0 / np.sqrt(128), rows=rows)
