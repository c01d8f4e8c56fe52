"""Seeded synthetic dictionaries and key/value vectors shaped like the FAD-KV workloads.

This module only draws inputs: unit-norm atoms and sparse mixtures of them, plus drifted
Gaussian vectors.  It holds none of the coder's arithmetic (no screening, pooling, pursuit,
ridge solve or adaptation) and is used alike by the HIP path's tests and benchmark and by the
CPU oracle's tests.  Real model K/V tensors and the benchmark datasets named on the pages are
not available; these draws stand in for them with the layer/head/head_dim shapes of the
models in the pages' tables (Llama-3.2-3B, Llama-3.1-8B, Qwen3-4B) and the Table 5
hyperparameters.

Recipe (per dictionary t, sub-seed = seed * 1000 + t):
  * atoms: isotropic workloads draw g ~ N(0, I_d) and normalise; anisotropic workloads draw a
    random r-dimensional subspace U and take normalise(U z + 0.1 w), z ~ N(0, I_r),
    w ~ N(0, I_d), which makes scores head-heavy like the Figure 1 diagnostics.  Atoms are
    normalised in fp32 and then rounded to the storage dtype.
  * planted rows: s_mix distinct atoms per row, coefficients N(0, 1), x = sum a_i d_i (stored
    atoms) plus N(0, noise_std^2) per coordinate, rounded to the storage dtype.  Support atoms
    come from a fixed random half of the dictionary with Zipf(1) popularity (anisotropic
    workloads) or uniformly from all atoms (isotropic ones), so part of the dictionary stays
    unused, as Figure 1 (c)-(d) reports after prefill.
  * drifted rows (a fraction drift_frac of each batch): Gaussian vectors with mean mu supported
    on the complement of U, rescaled so E||x||^2 = s_mix like the planted rows; mu moves
    linearly from mu0 to mu1 over a long run.  These code badly and trigger adaptation.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional

import numpy as np
import torch

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    num_dicts: int          # 2 * layers (key and value dictionary per layer) unless tiny
    kv_heads: int
    d: int                  # head_dim
    N: int                  # atoms per dictionary
    n: int                  # pool size
    s: int                  # sparsity
    dtype: str              # storage dtype of atoms and vectors
    seqs: int               # sequences per step
    tokens: int             # tokens per sequence per step
    s_mix: int              # atoms per planted vector
    noise_std: float
    drift_frac: float
    subspace: Optional[int]  # None: isotropic atoms
    seed: int
    steps: int = 1          # steps of a long run
    dict_seed: Optional[int] = None   # draw the dictionary of another workload

    @property
    def M(self) -> int:
        """Vectors per dictionary per step, rows ordered (head, sequence, token)."""
        return self.kv_heads * self.seqs * self.tokens

    @property
    def vectors_per_step(self) -> int:
        return self.num_dicts * self.M


WORKLOADS = {
    # one key dictionary, head_dim 64, 256 fp32 atoms, n=32, s=4, 512 planted 4-sparse vectors
    # with N(0, 0.01^2) noise, seed 0
    "tiny": Workload("tiny", 1, 1, 64, 256, 32, 4, "f32", 1, 512, 4, 0.01, 0.0, None, 0),
    # Llama-3.2-3B decode step: 28 layers x {K,V}, 8 KV heads, head_dim 128, N=4096 fp16,
    # n=256, s=8, 32 sequences x 1 token, 8-sparse mixes + 20% drifted vectors
    "llama3b_decode": Workload("llama3b_decode", 56, 8, 128, 4096, 256, 8, "f16", 32, 1, 8,
                               0.0, 0.20, 96, 1),
    # Llama-3.2-3B prefill: same dictionaries in bf16, one 8192-token sequence, mixes + noise
    "llama3b_prefill": Workload("llama3b_prefill", 56, 8, 128, 4096, 256, 8, "bf16", 1, 8192,
                                8, 0.05, 0.0, 96, 2, dict_seed=1),
    # Llama-3.1-8B decode step: 32 layers, N=8192, n=512, s=16, 64 sequences x 1 token
    "llama8b_decode": Workload("llama8b_decode", 64, 8, 128, 8192, 512, 16, "f16", 64, 1, 16,
                               0.0, 0.20, 96, 3),
    # Qwen3-4B long run: 36 layers, N=4096 bf16, 16384-token prefill, then 1024 decode steps
    # at 16 sequences with linearly drifting inputs
    "qwen4b_long_prefill": Workload("qwen4b_long_prefill", 72, 8, 128, 4096, 256, 8, "bf16", 1,
                                    16384, 8, 0.05, 0.0, 96, 4),
    "qwen4b_long_decode": Workload("qwen4b_long_decode", 72, 8, 128, 4096, 256, 8, "bf16", 16, 1,
                                   8, 0.0, 0.20, 96, 4, steps=1024),
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


class SyntheticKV:
    """Dictionaries and per-step batches for one workload, on ``device``."""

    def __init__(self, w: Workload, device="cpu", num_dicts: Optional[int] = None):
        self.w = w
        self.device = torch.device(device)
        self.T = w.num_dicts if num_dicts is None else num_dicts
        self._state = [self._dict_state(t) for t in range(self.T)]

    # -- per-dictionary fixed state (subspace, popular half, drift means) -------------------
    def _dict_state(self, t: int):
        w = self.w
        seed = (w.dict_seed if w.dict_seed is not None else w.seed) * 1000 + t
        g = _gen(seed, "cpu")
        d = w.d
        st = {}
        if w.subspace is not None:
            q, _ = torch.linalg.qr(torch.randn(d, d, generator=g, dtype=torch.float64))
            st["U"] = q[:, : w.subspace].to(torch.float32)
            st["Uperp"] = q[:, w.subspace:].to(torch.float32)
            half = torch.randperm(w.N, generator=g)[: w.N // 2]
            st["support_atoms"] = half
            ranks = torch.arange(1, half.numel() + 1, dtype=torch.float64)
            st["weights"] = (1.0 / ranks).to(torch.float32)
        else:
            st["support_atoms"] = torch.arange(w.N)
            st["weights"] = torch.ones(w.N, dtype=torch.float32)
        # drift means live in the complement of U (or anywhere, isotropic case)
        basis = st.get("Uperp")
        k = basis.shape[1] if basis is not None else d
        m0 = torch.randn(k, generator=g)
        m1 = torch.randn(k, generator=g)
        st["mu0"] = m0 / m0.norm()
        st["mu1"] = m1 / m1.norm()
        st["atom_seed"] = seed
        return st

    def atoms(self) -> torch.Tensor:
        """[T][N][d] unit-norm atoms in the storage dtype (normalised in fp32, then rounded)."""
        w = self.w
        out = torch.empty(self.T, w.N, w.d, dtype=TORCH_DTYPES[w.dtype], device=self.device)
        for t in range(self.T):
            st = self._state[t]
            g = _gen(st["atom_seed"] * 7 + 1, "cpu")
            if w.subspace is not None:
                z = torch.randn(w.N, w.subspace, generator=g)
                noise = torch.randn(w.N, w.d, generator=g)
                a = z @ st["U"].T + 0.1 * noise
            else:
                a = torch.randn(w.N, w.d, generator=g)
            a = a / a.norm(dim=1, keepdim=True)
            out[t] = a.to(self.device).to(out.dtype)
        return out

    # -- one step of vectors ----------------------------------------------------------------
    def batch(self, atoms: torch.Tensor, step: int = 0, M: Optional[int] = None,
              drift_frac: Optional[float] = None, noise_std: Optional[float] = None,
              support_limit: Optional[int] = None) -> torch.Tensor:
        """[T][M][d] vectors in the storage dtype drawn against the given atoms.

        ``support_limit`` restricts planted supports to atoms [0, support_limit) (test variants
        that need unused atoms in an isotropic dictionary).
        """
        w = self.w
        M = w.M if M is None else M
        drift_frac = w.drift_frac if drift_frac is None else drift_frac
        noise_std = w.noise_std if noise_std is None else noise_std
        dev = self.device
        out = torch.empty(self.T, M, w.d, dtype=atoms.dtype, device=dev)
        frac_t = (step / max(1, w.steps - 1)) if w.steps > 1 else 0.0
        for t in range(self.T):
            st = self._state[t]
            g = _gen(st["atom_seed"] * 1_000_003 + 104_729 * (step + 1), dev)
            A = atoms[t].to(torch.float32)
            if support_limit is not None:
                pop = torch.arange(support_limit, device=dev)
                wts = torch.ones(support_limit, device=dev)
            else:
                pop = st["support_atoms"].to(dev)
                wts = st["weights"].to(dev)
            sel = torch.multinomial(wts.expand(M, -1).contiguous(), w.s_mix, replacement=False,
                                    generator=g)
            support = pop[sel]                                  # [M][s_mix]
            coef = torch.randn(M, w.s_mix, generator=g, device=dev)
            x = torch.einsum("mk,mkd->md", coef, A[support])
            if noise_std > 0:
                x = x + noise_std * torch.randn(M, w.d, generator=g, device=dev)
            n_drift = int(round(drift_frac * M))
            if n_drift > 0:
                rows = torch.randperm(M, generator=g, device=dev)[:n_drift]
                mu = ((1 - frac_t) * st["mu0"] + frac_t * st["mu1"]).to(dev)
                mu = mu / mu.norm()
                if "Uperp" in st:
                    B = st["Uperp"].to(dev)                     # [d][k]
                    k = B.shape[1]
                    gz = torch.randn(n_drift, k, generator=g, device=dev)
                    y = (2.0 * mu + gz * (4.0 / k) ** 0.5) @ B.T
                else:
                    gz = torch.randn(n_drift, w.d, generator=g, device=dev)
                    y = 2.0 * mu + gz * (4.0 / w.d) ** 0.5
                y = y * (w.s_mix ** 0.5 / 8.0 ** 0.5)
                x[rows] = y
            out[t] = x.to(out.dtype)
        return out


def usage_zeros(w: Workload, T: Optional[int] = None, device="cpu") -> torch.Tensor:
    return torch.zeros((w.num_dicts if T is None else T), w.N, dtype=torch.int32, device=device)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a stored tensor (every f32/f16/bf16 value is exact in f64)."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def variant(w: Workload, **kw) -> Workload:
    return replace(w, **kw)
