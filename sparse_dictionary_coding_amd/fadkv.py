"""Thin ctypes binding of libfadkv (include/fadkv.h), for torch tensors on the GPU.

Argument marshalling only: shapes and dtypes are checked, device pointers and torch's current
HIP stream are passed to the C functions of the same names, and a negative status raises
FadkvError.  Every step of the coder runs in the library's HIP kernels; there is no fallback.
The library is loaded on first use (after torch, so that it binds to torch's HIP runtime) and
a missing library raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfadkv.so")

FADKV_OK = 0
FADKV_F32, FADKV_F16, FADKV_BF16 = 0, 1, 2
FADKV_SELECT_GM, FADKV_SELECT_PL = 0, 1
FLAG_TRIGGER, FLAG_REPLACED, FLAG_EXHAUSTED, FLAG_NONFINITE = 0x01, 0x02, 0x04, 0x08

_DT = {torch.float32: FADKV_F32, torch.float16: FADKV_F16, torch.bfloat16: FADKV_BF16}
_TORCH_DT = {v: k for k, v in _DT.items()}
_SELECT = {"gm": FADKV_SELECT_GM, "pl": FADKV_SELECT_PL}


class FadkvError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed with status {status}: {fadkv_status_string(status)}")
        self.status = status


class fadkv_dict(ctypes.Structure):
    _fields_ = [("num_dicts", ctypes.c_int32), ("N", ctypes.c_int32), ("d", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("atoms", ctypes.c_void_p), ("usage", ctypes.c_void_p)]


class fadkv_params(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("s", ctypes.c_int32), ("ridge_abs", ctypes.c_float),
                ("ridge_rel", ctypes.c_float), ("delta_key", ctypes.c_float),
                ("delta_value", ctypes.c_float), ("tau_c", ctypes.c_uint32),
                ("select", ctypes.c_int32)]


class fadkv_codes(ctypes.Structure):
    _fields_ = [("idx", ctypes.c_void_p), ("coef", ctypes.c_void_p), ("relerr", ctypes.c_void_p),
                ("flags", ctypes.c_void_p)]


_lib_handle = None


def lib() -> ctypes.CDLL:
    """The loaded libfadkv.so (raises if it has not been built)."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_dictionary_coding_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        h.fadkv_abi_version.restype = ctypes.c_int
        h.fadkv_status_string.restype = ctypes.c_char_p
        h.fadkv_status_string.argtypes = [ctypes.c_int]
        h.fadkv_workspace_bytes.restype = ctypes.c_int
        h.fadkv_workspace_bytes.argtypes = [P(fadkv_dict), P(fadkv_params), ctypes.c_int64,
                                            P(ctypes.c_size_t)]
        h.fadkv_encode.restype = ctypes.c_int
        h.fadkv_encode.argtypes = [P(fadkv_dict), P(fadkv_params), ctypes.c_void_p, ctypes.c_int64,
                                   P(fadkv_codes), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        h.fadkv_encode_noalloc.restype = ctypes.c_int
        h.fadkv_encode_noalloc.argtypes = [P(fadkv_dict), P(fadkv_params), ctypes.c_void_p,
                                           ctypes.c_int64, P(fadkv_codes), ctypes.c_void_p]
        h.fadkv_screen.restype = ctypes.c_int
        h.fadkv_screen.argtypes = [P(fadkv_dict), P(fadkv_params), ctypes.c_void_p, ctypes.c_int64,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p]
        h.fadkv_select_support.restype = ctypes.c_int
        h.fadkv_select_support.argtypes = [P(fadkv_dict), P(fadkv_params), ctypes.c_void_p,
                                           ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p, P(fadkv_codes), ctypes.c_void_p]
        h.fadkv_adapt.restype = ctypes.c_int
        h.fadkv_adapt.argtypes = [P(fadkv_dict), P(fadkv_params), ctypes.c_void_p, ctypes.c_int64,
                                  P(fadkv_codes), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                  ctypes.c_void_p]
        h.fadkv_reconstruct.restype = ctypes.c_int
        h.fadkv_reconstruct.argtypes = [P(fadkv_dict), ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p,
                                        ctypes.c_int32, ctypes.c_void_p]
        h.fadkv_adapt_append.restype = ctypes.c_int
        h.fadkv_adapt_append.argtypes = [P(fadkv_dict), P(fadkv_params), ctypes.c_void_p,
                                         ctypes.c_int64, P(fadkv_codes), ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                         ctypes.c_void_p]
        h.fadkv_omp_workspace_bytes.restype = ctypes.c_int
        h.fadkv_omp_workspace_bytes.argtypes = [P(fadkv_dict), P(fadkv_params), ctypes.c_int64,
                                                P(ctypes.c_size_t)]
        h.fadkv_encode_omp.restype = ctypes.c_int
        h.fadkv_encode_omp.argtypes = [P(fadkv_dict), P(fadkv_params), ctypes.c_void_p,
                                       ctypes.c_int64, P(fadkv_codes), ctypes.c_void_p,
                                       ctypes.c_size_t, ctypes.c_void_p]
        h.fadkv_attend_workspace_bytes.restype = ctypes.c_int
        h.fadkv_attend_workspace_bytes.argtypes = [P(fadkv_dict), ctypes.c_int64, ctypes.c_int32,
                                                   P(ctypes.c_size_t)]
        h.fadkv_attend.restype = ctypes.c_int
        h.fadkv_attend.argtypes = [P(fadkv_dict), ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                   ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_float,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.c_void_p]
        _lib_handle = h
    return _lib_handle


def fadkv_status_string(status: int) -> str:
    return lib().fadkv_status_string(int(status)).decode()


def fadkv_abi_version() -> int:
    return int(lib().fadkv_abi_version())


@dataclass(frozen=True)
class Params:
    """fadkv_params (defaults: Table 5, 3B/4B column)."""

    n: int = 256
    s: int = 8
    ridge_abs: float = 1e-4
    ridge_rel: float = 0.20
    delta_key: float = 0.50
    delta_value: float = 0.70
    tau_c: int = 1
    select: str = "gm"

    def c(self) -> fadkv_params:
        return fadkv_params(self.n, self.s, self.ridge_abs, self.ridge_rel, self.delta_key,
                            self.delta_value, self.tau_c, _SELECT[self.select])


@dataclass
class Codes:
    idx: torch.Tensor      # int32 [num_dicts][M][s]
    coef: torch.Tensor     # float32 [num_dicts][M][s]
    relerr: torch.Tensor   # float32 [num_dicts][M]
    flags: torch.Tensor    # uint8 [num_dicts][M]

    @staticmethod
    def empty(num_dicts: int, M: int, s: int, device) -> "Codes":
        return Codes(torch.empty(num_dicts, M, s, dtype=torch.int32, device=device),
                     torch.empty(num_dicts, M, s, dtype=torch.float32, device=device),
                     torch.empty(num_dicts, M, dtype=torch.float32, device=device),
                     torch.empty(num_dicts, M, dtype=torch.uint8, device=device))

    def c(self) -> fadkv_codes:
        return fadkv_codes(self.idx.data_ptr(), self.coef.data_ptr(), self.relerr.data_ptr(),
                           self.flags.data_ptr())


def _check(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _dict(atoms: torch.Tensor, usage: Optional[torch.Tensor] = None) -> fadkv_dict:
    _check(atoms, "atoms")
    if atoms.dim() != 3 or atoms.dtype not in _DT:
        raise ValueError("atoms must be [num_dicts][N][d] float32/float16/bfloat16")
    T, N, d = atoms.shape
    if usage is not None:
        _check(usage, "usage", torch.int32, (T, N))
    return fadkv_dict(T, N, d, _DT[atoms.dtype], atoms.data_ptr(),
                      usage.data_ptr() if usage is not None else None)


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def fadkv_workspace_bytes(atoms: torch.Tensor, params: Params, M: int) -> int:
    T, N, d = atoms.shape
    dd = fadkv_dict(T, N, d, _DT[atoms.dtype], None, None)
    out = ctypes.c_size_t(0)
    st = lib().fadkv_workspace_bytes(ctypes.byref(dd), ctypes.byref(params.c()), int(M),
                                     ctypes.byref(out))
    if st != FADKV_OK:
        raise FadkvError("fadkv_workspace_bytes", st)
    return int(out.value)


def make_workspace(atoms: torch.Tensor, params: Params, M: int) -> torch.Tensor:
    return torch.empty(max(1, fadkv_workspace_bytes(atoms, params, M)), dtype=torch.uint8,
                       device=atoms.device)


def fadkv_encode(atoms: torch.Tensor, X: torch.Tensor, params: Params,
                 out: Optional[Codes] = None, workspace: Optional[torch.Tensor] = None,
                 stream=None) -> Codes:
    """Encode X[t][m] against atoms[t]; returns (or fills) the codes."""
    dd = _dict(atoms)
    T, N, d = atoms.shape
    _check(X, "X", atoms.dtype)
    if X.dim() != 3 or X.shape[0] != T or X.shape[2] != d:
        raise ValueError(f"X must be [{T}][M][{d}]")
    M = X.shape[1]
    if out is None:
        out = Codes.empty(T, M, params.s, atoms.device)
    if workspace is None:
        workspace = make_workspace(atoms, params, M)
    st = lib().fadkv_encode(ctypes.byref(dd), ctypes.byref(params.c()), X.data_ptr(), M,
                            ctypes.byref(out.c()), workspace.data_ptr(), workspace.numel(),
                            _stream(stream))
    if st != FADKV_OK:
        raise FadkvError("fadkv_encode", st)
    return out


NOALLOC_SCRATCH_BYTES = 128 << 20    # FADKV_NOALLOC_SCRATCH_BYTES
FADKV_ERR_SCRATCH = -6


def fadkv_encode_noalloc(atoms: torch.Tensor, X: torch.Tensor, params: Params,
                         out: Optional[Codes] = None, stream=None) -> Codes:
    """fadkv_encode with the library's static per-GPU scratch instead of a workspace (for
    callers that cannot allocate); `out` is the caller's, allocated here only when not given.
    Calls that overlap on one GPU race on that scratch."""
    dd = _dict(atoms)
    T, N, d = atoms.shape
    _check(X, "X", atoms.dtype)
    if X.dim() != 3 or X.shape[0] != T or X.shape[2] != d:
        raise ValueError(f"X must be [{T}][M][{d}]")
    M = X.shape[1]
    if out is None:
        out = Codes.empty(T, M, params.s, atoms.device)
    st = lib().fadkv_encode_noalloc(ctypes.byref(dd), ctypes.byref(params.c()), X.data_ptr(), M,
                                    ctypes.byref(out.c()), _stream(stream))
    if st != FADKV_OK:
        raise FadkvError("fadkv_encode_noalloc", st)
    return out


@dataclass
class Pool:
    idx: torch.Tensor      # int16 storage of uint16 atom indices [num_dicts][M][n]
    score: torch.Tensor    # float32 [num_dicts][M][n]
    status: torch.Tensor   # uint8 [num_dicts][M]: 0 encoded, 1 zero vector, 2 non-finite

    @staticmethod
    def empty(num_dicts: int, M: int, n: int, device) -> "Pool":
        return Pool(torch.empty(num_dicts, M, n, dtype=torch.int16, device=device),
                    torch.empty(num_dicts, M, n, dtype=torch.float32, device=device),
                    torch.empty(num_dicts, M, dtype=torch.uint8, device=device))

    def atom_indices(self) -> torch.Tensor:
        """Pool indices as int64 (the uint16 values)."""
        return self.idx.to(torch.int64) & 0xFFFF


def fadkv_screen(atoms: torch.Tensor, X: torch.Tensor, params: Params,
                 out: Optional[Pool] = None, stream=None) -> Pool:
    """Scores and Top-n pool of every vector (first stage of fadkv_encode)."""
    dd = _dict(atoms)
    T, N, d = atoms.shape
    _check(X, "X", atoms.dtype)
    M = X.shape[1]
    if out is None:
        out = Pool.empty(T, M, params.n, atoms.device)
    st = lib().fadkv_screen(ctypes.byref(dd), ctypes.byref(params.c()), X.data_ptr(), M,
                            out.idx.data_ptr(), out.score.data_ptr(), out.status.data_ptr(),
                            _stream(stream))
    if st != FADKV_OK:
        raise FadkvError("fadkv_screen", st)
    return out


def fadkv_select_support(atoms: torch.Tensor, X: torch.Tensor, params: Params, pool: Pool,
                         out: Optional[Codes] = None, stream=None) -> Codes:
    """Support, ridge coefficients and residual from a screened pool (second stage)."""
    dd = _dict(atoms)
    T, N, d = atoms.shape
    _check(X, "X", atoms.dtype)
    M = X.shape[1]
    if out is None:
        out = Codes.empty(T, M, params.s, atoms.device)
    st = lib().fadkv_select_support(ctypes.byref(dd), ctypes.byref(params.c()), X.data_ptr(), M,
                                    pool.idx.data_ptr(), pool.score.data_ptr(),
                                    pool.status.data_ptr(), ctypes.byref(out.c()), _stream(stream))
    if st != FADKV_OK:
        raise FadkvError("fadkv_select_support", st)
    return out


def fadkv_adapt(atoms: torch.Tensor, usage: torch.Tensor, X: torch.Tensor, codes: Codes,
                params: Params, replaced: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Commit this step's codes and overwrite inactive atoms in place; returns `replaced`."""
    dd = _dict(atoms, usage)
    T, N, d = atoms.shape
    _check(X, "X", atoms.dtype)
    M = X.shape[1]
    if replaced is None:
        replaced = torch.empty(T, M, dtype=torch.int32, device=atoms.device)
    if workspace is None:
        workspace = make_workspace(atoms, params, M)
    st = lib().fadkv_adapt(ctypes.byref(dd), ctypes.byref(params.c()), X.data_ptr(), M,
                           ctypes.byref(codes.c()), replaced.data_ptr(), workspace.data_ptr(),
                           workspace.numel(), _stream(stream))
    if st != FADKV_OK:
        raise FadkvError("fadkv_adapt", st)
    return replaced


def fadkv_reconstruct(atoms: torch.Tensor, idx: torch.Tensor, coef: torch.Tensor,
                      out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    dd = _dict(atoms)
    T, N, d = atoms.shape
    _check(idx, "idx", torch.int32)
    _check(coef, "coef", torch.float32, idx.shape)
    M, s = idx.shape[1], idx.shape[2]
    if out is None:
        out = torch.empty(T, M, d, dtype=out_dtype or atoms.dtype, device=atoms.device)
    _check(out, "out", None, (T, M, d))
    st = lib().fadkv_reconstruct(ctypes.byref(dd), idx.data_ptr(), coef.data_ptr(), s, M,
                                 out.data_ptr(), _DT[out.dtype], _stream(stream))
    if st != FADKV_OK:
        raise FadkvError("fadkv_reconstruct", st)
    return out


def fadkv_attend_workspace_bytes(atoms: torch.Tensor, R: int, G: int) -> int:
    T, N, d = atoms.shape
    dd = fadkv_dict(T, N, d, _DT[atoms.dtype], None, None)
    out = ctypes.c_size_t(0)
    st = lib().fadkv_attend_workspace_bytes(ctypes.byref(dd), int(R), int(G), ctypes.byref(out))
    if st != FADKV_OK:
        raise FadkvError("fadkv_attend_workspace_bytes", st)
    return int(out.value)


def fadkv_attend(atoms: torch.Tensor, layer: int, k_idx: torch.Tensor, k_coef: torch.Tensor,
                 v_idx: torch.Tensor, v_coef: torch.Tensor, lens: torch.Tensor, q: torch.Tensor,
                 scale: float, out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Decode attention of q [R][G][d] over the sparse-coded keys/values of `layer` (codes
    [R][T][s], lens [R]); returns (or fills) out [R][G][d] fp32."""
    dd = _dict(atoms)
    _check(k_idx, "k_idx", torch.int32)
    R, T, s = k_idx.shape
    _check(k_coef, "k_coef", torch.float32, (R, T, s))
    _check(v_idx, "v_idx", torch.int32, (R, T, s))
    _check(v_coef, "v_coef", torch.float32, (R, T, s))
    _check(lens, "lens", torch.int32, (R,))
    _check(q, "q", atoms.dtype)
    if q.dim() != 3 or q.shape[0] != R or q.shape[2] != atoms.shape[2]:
        raise ValueError(f"q must be [{R}][G][{atoms.shape[2]}]")
    G = q.shape[1]
    if out is None:
        out = torch.empty(R, G, atoms.shape[2], dtype=torch.float32, device=atoms.device)
    _check(out, "out", torch.float32, (R, G, atoms.shape[2]))
    if workspace is None:
        workspace = torch.empty(max(1, fadkv_attend_workspace_bytes(atoms, R, G)),
                                dtype=torch.uint8, device=atoms.device)
    st = lib().fadkv_attend(ctypes.byref(dd), int(layer), int(s), k_idx.data_ptr(),
                            k_coef.data_ptr(), v_idx.data_ptr(), v_coef.data_ptr(),
                            lens.data_ptr(), int(R), int(T), q.data_ptr(), int(G), float(scale),
                            out.data_ptr(), workspace.data_ptr(), workspace.numel(),
                            _stream(stream))
    if st != FADKV_OK:
        raise FadkvError("fadkv_attend", st)
    return out


def fadkv_adapt_append(atoms: torch.Tensor, usage: torch.Tensor, X: torch.Tensor, codes: Codes,
                       params: Params, n_atoms: torch.Tensor,
                       replaced: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Append-only growth commit: atoms [num_dicts][capacity][d] with n_atoms [num_dicts]
    (int32, advanced in place) slots in use.  Returns replaced [num_dicts][M]."""
    dd = _dict(atoms, usage)
    T, N, d = atoms.shape
    _check(X, "X", atoms.dtype)
    M = X.shape[1]
    _check(n_atoms, "n_atoms", torch.int32, (T,))
    if replaced is None:
        replaced = torch.empty(T, M, dtype=torch.int32, device=atoms.device)
    _check(replaced, "replaced", torch.int32, (T, M))
    if workspace is None:
        workspace = make_workspace(atoms, params, M)
    st = lib().fadkv_adapt_append(ctypes.byref(dd), ctypes.byref(params.c()), X.data_ptr(), M,
                                  ctypes.byref(codes.c()), replaced.data_ptr(), n_atoms.data_ptr(),
                                  workspace.data_ptr(), workspace.numel(), _stream(stream))
    if st != FADKV_OK:
        raise FadkvError("fadkv_adapt_append", st)
    return replaced


def fadkv_omp_workspace_bytes(atoms: torch.Tensor, params: Params, M: int) -> int:
    T, N, d = atoms.shape
    dd = fadkv_dict(T, N, d, _DT[atoms.dtype], None, None)
    out = ctypes.c_size_t(0)
    st = lib().fadkv_omp_workspace_bytes(ctypes.byref(dd), ctypes.byref(params.c()), int(M),
                                         ctypes.byref(out))
    if st != FADKV_OK:
        raise FadkvError("fadkv_omp_workspace_bytes", st)
    return out.value


def fadkv_encode_omp(atoms: torch.Tensor, X: torch.Tensor, params: Params,
                     out: Optional[Codes] = None, workspace: Optional[torch.Tensor] = None,
                     stream=None) -> Codes:
    """Full-dictionary greedy yardstick (every atom a candidate); codes as fadkv_encode."""
    dd = _dict(atoms, None)
    T, N, d = atoms.shape
    _check(X, "X", atoms.dtype)
    M = X.shape[1]
    if out is None:
        out = Codes.empty(T, M, params.s, atoms.device)
    if workspace is None:
        workspace = torch.empty(max(1, fadkv_omp_workspace_bytes(atoms, params, M)),
                                dtype=torch.uint8, device=atoms.device)
    st = lib().fadkv_encode_omp(ctypes.byref(dd), ctypes.byref(params.c()), X.data_ptr(), M,
                                ctypes.byref(out.c()), workspace.data_ptr(), workspace.numel(),
                                _stream(stream))
    if st != FADKV_OK:
        raise FadkvError("fadkv_encode_omp", st)
    return out
