"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI and compare its
outputs with the CPU oracle on the same seeded inputs.

Comparison rules (a vector's oracle near-tie flag decides which one applies):
  * decisions without a near-tie must match exactly: selected atoms in selection order, the
    trigger bit, adaptation slots;
  * at a near-tie the GPU's choice must be a valid one (oracle.replay_support), and its
    coefficients/error are compared with the oracle's on the GPU's own support;
  * coefficients agree within 1e-4 relative (norm over the code), relative errors within 1e-4
    relative: the GPU accumulates in fp32 (scores, Cholesky, residual), the oracle in fp64, and
    the fp32 error of these O(d)-term sums is ~1e-6 relative, so 1e-4 leaves two decades.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

import oracle
from oracle import OracleParams
from oracle.fadkv_oracle import FLAG_NEAR_TIE, FLAG_NONFINITE, FLAG_TRIGGER, TIE_DELTA
from sparse_dictionary_coding_amd import fadkv
from sparse_dictionary_coding_amd.synth import to_f64

COEF_RTOL = 1e-4
ERR_RTOL = 1e-4
ABS_FLOOR = 1e-6

_DT_NAME = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}


def dtype_name(t: torch.Tensor) -> str:
    return _DT_NAME[t.dtype]


def f32(v: float) -> float:
    """The float32 value the C ABI will see for a parameter."""
    return float(np.float32(v))


def oracle_params(p: fadkv.Params) -> OracleParams:
    return OracleParams(n=p.n, s=p.s, ridge_abs=f32(p.ridge_abs), ridge_rel=f32(p.ridge_rel),
                        delta_key=f32(p.delta_key), delta_value=f32(p.delta_value),
                        tau_c=p.tau_c, select=p.select)


def codes_to_numpy(c: fadkv.Codes):
    return (c.idx.cpu().numpy(), c.coef.cpu().numpy().astype(np.float64),
            c.relerr.cpu().numpy().astype(np.float64), c.flags.cpu().numpy())


def oracle_codes_to_gpu(oc: oracle.Codes, device) -> fadkv.Codes:
    return fadkv.Codes(torch.from_numpy(oc.idx.astype(np.int32)).to(device),
                       torch.from_numpy(oc.coef.astype(np.float32)).to(device),
                       torch.from_numpy(oc.relerr.astype(np.float32)).to(device),
                       torch.from_numpy((oc.flags & np.uint8(0xFF ^ FLAG_NEAR_TIE)).astype(np.uint8)).to(device))


@dataclass
class Report:
    vectors: int = 0
    exact: int = 0
    near_tie: int = 0
    nonfinite: int = 0
    failures: list = field(default_factory=list)

    def check(self, max_report=10):
        assert not self.failures, (f"{len(self.failures)} parity failures of {self.vectors} "
                                   f"vectors, first: " + "; ".join(self.failures[:max_report]))


def _close(a, b, rtol):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.linalg.norm(a - b) <= rtol * np.linalg.norm(b) + ABS_FLOOR


def compare_vector(rep: Report, where: str, D, x, gi, gc, ge, gf, oc: oracle.VectorCode,
                   p: OracleParams, delta: float, pool=None):
    """Compare one vector's GPU code with the oracle's.  ``pool``, when given, is the candidate
    pool the GPU screened for this vector: a near-tie choice is then replayed inside that pool
    (the pool must itself be a valid Top-n, and every greedy pick the best of its own pool)."""
    rep.vectors += 1
    if oc.flags & FLAG_NONFINITE:
        rep.nonfinite += 1
        if not (gf & FLAG_NONFINITE) or np.any(gi != -1) or not np.isnan(ge):
            rep.failures.append(f"{where}: non-finite input not flagged as such")
        return
    if oc.ties == 0:
        rep.exact += 1
        if not np.array_equal(gi, oc.idx):
            rep.failures.append(f"{where}: idx {gi.tolist()} != oracle {oc.idx.tolist()}")
            return
        if not _close(gc, oc.coef, COEF_RTOL):
            rep.failures.append(f"{where}: coef {gc} vs {oc.coef}")
        if abs(ge - oc.relerr) > ERR_RTOL * oc.relerr + ABS_FLOOR:
            rep.failures.append(f"{where}: relerr {ge} vs {oc.relerr}")
        if (gf & FLAG_TRIGGER) != (oc.flags & FLAG_TRIGGER):
            rep.failures.append(f"{where}: trigger {gf & 1} vs {oc.flags & 1}")
        return
    rep.near_tie += 1
    valid, why, c, e = oracle.replay_support(D, x, gi, p, pool=pool)
    if not valid:
        rep.failures.append(f"{where}: near-tie choice invalid: {why}")
        return
    if not _close(gc[: len(c)], c, COEF_RTOL):
        rep.failures.append(f"{where}: coef {gc} vs replay {c}")
    if abs(ge - e) > ERR_RTOL * e + ABS_FLOOR:
        rep.failures.append(f"{where}: relerr {ge} vs replay {e}")
    if oc.ties & TIE_DELTA:
        if bool(gf & FLAG_TRIGGER) != (ge > delta):
            rep.failures.append(f"{where}: trigger bit inconsistent with its own error")
    elif (gf & FLAG_TRIGGER) != (oc.flags & FLAG_TRIGGER):
        rep.failures.append(f"{where}: trigger {gf & 1} vs {oc.flags & 1}")


def compare_encode(atoms_f64, X_f64, gpu, p: OracleParams, rows=None, dict_ids=None,
                   oracle_codes: oracle.Codes | None = None,
                   pools=None) -> tuple[Report, oracle.Codes]:
    """Compare GPU codes (numpy tuple) with the oracle on every (or the listed) rows.

    rows: iterable of (t, m); dict_ids gives the dictionary number of slice t (delta parity);
    pools: the GPU's candidate pools [T][M][n] (pool_from_workspace), used at near-ties.
    Returns the report and the oracle's codes for all compared rows (full arrays when rows is
    None).
    """
    gi, gc, ge, gf = gpu
    T, M = X_f64.shape[0], X_f64.shape[1]
    ids = list(range(T)) if dict_ids is None else list(dict_ids)
    rep = Report()
    if oracle_codes is None and rows is None:
        oracle_codes = oracle.encode(atoms_f64, X_f64, p, ids)
    pairs = [(t, m) for t in range(T) for m in range(M)] if rows is None else list(rows)
    for (t, m) in pairs:
        delta = p.delta(ids[t])
        if oracle_codes is not None:
            oc = oracle.VectorCode(oracle_codes.idx[t, m], oracle_codes.coef[t, m],
                                   oracle_codes.relerr[t, m], int(oracle_codes.flags[t, m]),
                                   int(oracle_codes.ties[t, m]))
        else:
            oc = oracle.encode_vector(atoms_f64[t], X_f64[t, m], p, delta)
        compare_vector(rep, f"dict {t} row {m}", atoms_f64[t], X_f64[t, m], gi[t, m], gc[t, m],
                       ge[t, m], int(gf[t, m]), oc, p, delta,
                       pool=None if pools is None else pools[t, m])
    return rep, oracle_codes


def gpu_encode(atoms: torch.Tensor, X: torch.Tensor, p: fadkv.Params, workspace=None):
    codes = fadkv.fadkv_encode(atoms, X, p, workspace=workspace)
    torch.cuda.synchronize()
    return codes


def pool_from_workspace(ws: torch.Tensor, T: int, M: int, n: int):
    """The candidate pools the screening kernel left at the head of the workspace
    (uint16 [T*M][n] indices, then 256-byte aligned float32 [T*M][n] scores)."""
    G = T * M
    nb = G * n * 2
    idx = ws[:nb].view(torch.int16).to(torch.int32).cpu().numpy() & 0xFFFF
    off = (nb + 255) // 256 * 256
    sig = ws[off: off + G * n * 4].view(torch.float32).cpu().numpy()
    return idx.reshape(T, M, n), sig.reshape(T, M, n)


def pool_rows_from_workspace(ws: torch.Tensor, T: int, M: int, n: int, rows):
    """The GPU's candidate pools of the listed rows (t, m) only, from the workspace head (see
    pool_from_workspace), as {(t, m): int64 atom indices}."""
    idx = ws[: T * M * n * 2].view(torch.int16).view(T, M, n)
    return {(t, m): idx[t, m].to(torch.int64).cpu().numpy() & 0xFFFF for (t, m) in rows}


def to_host(t: torch.Tensor) -> np.ndarray:
    return to_f64(t)


def gpu_codes_as_oracle(gi, gc, ge, gf) -> oracle.Codes:
    """The GPU's codes (numpy arrays from codes_to_numpy) as oracle Codes, so that the oracle
    can commit exactly the supports and trigger bits the GPU produced."""
    return oracle.Codes(np.array(gi, np.int32, copy=True), np.array(gc, np.float64, copy=True),
                        np.array(ge, np.float64, copy=True), np.array(gf, np.uint8, copy=True),
                        np.zeros(np.shape(gf), np.uint8))


def check_commit(where: str, A_before, U_before, X, gpu_before, op: OracleParams, dtype: str,
                 A_after, U_after, replaced, gpu_after):
    """The adaptation commit of one step, exactly: the oracle commits the GPU's own codes
    (supports and trigger bits as the GPU encoded them) from the GPU's step-start atoms and
    usage; the GPU's replacements, usage counters, new atoms and rewritten codes must equal the
    oracle's.  Adaptation reads nothing else of the codes, so this holds whatever near-ties the
    encode met.  Returns (number of replacements, number of exhausted rows)."""
    oc = gpu_codes_as_oracle(*gpu_before)
    na, nu, ncodes, orep = oracle.adapt(A_before, U_before, X, oc, op, dtype)
    gi, gc, ge, gf = gpu_after
    assert np.array_equal(replaced, orep), f"{where}: replacements differ"
    assert np.array_equal(np.asarray(U_after, np.int64), nu), f"{where}: usage counters differ"
    assert np.array_equal(A_after, na), f"{where}: new atoms differ"
    assert np.array_equal(gi, ncodes.idx), f"{where}: rewritten code indices differ"
    assert np.array_equal(gf, ncodes.flags), f"{where}: flags differ"
    np.testing.assert_allclose(gc, ncodes.coef, rtol=1e-6, atol=1e-7, err_msg=where)
    np.testing.assert_allclose(ge, ncodes.relerr, rtol=1e-6, atol=1e-7, err_msg=where)
    from oracle.fadkv_oracle import FLAG_EXHAUSTED
    return int(np.sum(orep >= 0)), int(np.sum((ncodes.flags & FLAG_EXHAUSTED) != 0))
