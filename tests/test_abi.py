"""C-ABI checks that need no GPU: the library loads, exports every function include/fadkv.h
declares, sizes workspaces, and rejects bad arguments on the host before enqueuing anything.

Invalid calls use fake (never dereferenced) device addresses: argument checking returns before
any HIP call, so no GPU is touched.
"""
import ctypes
import os
import re

import pytest

from sparse_dictionary_coding_amd import fadkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fadkv.h")

pytestmark = pytest.mark.skipif(not os.path.exists(fadkv.LIB_PATH),
                                reason="libfadkv.so not built (run __graft_entry__.build())")

FAKE = 0x7F0000100000          # 256-byte aligned, never dereferenced by the host checks


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fadkv_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary_calls():
    names = declared_functions()
    for fn in ("fadkv_encode", "fadkv_adapt", "fadkv_adapt_append", "fadkv_reconstruct",
               "fadkv_workspace_bytes", "fadkv_attend", "fadkv_attend_workspace_bytes",
               "fadkv_status_string", "fadkv_abi_version"):
        assert fn in names


def test_library_exports_every_declared_function():
    h = ctypes.CDLL(fadkv.LIB_PATH)
    for fn in declared_functions():
        assert hasattr(h, fn), f"{fn} declared in fadkv.h but not exported"


def test_abi_version_and_status_strings():
    assert fadkv.fadkv_abi_version() == 1
    for st in (0, -1, -2, -3, -4, -5):
        assert fadkv.fadkv_status_string(st) and fadkv.fadkv_status_string(st) != "unknown status"
    assert fadkv.fadkv_status_string(-99) == "unknown status"


def _dict(num_dicts=2, N=1024, d=128, dtype=fadkv.FADKV_F16, atoms=FAKE, usage=FAKE):
    return fadkv.fadkv_dict(num_dicts, N, d, dtype, atoms, usage)


def _params(**kw):
    base = dict(n=256, s=8, ridge_abs=1e-4, ridge_rel=0.2, delta_key=0.5, delta_value=0.7,
                tau_c=1, select=0)
    base.update(kw)
    return fadkv.fadkv_params(**base)


def _ws(dd, pp, M):
    out = ctypes.c_size_t(0)
    st = fadkv.lib().fadkv_workspace_bytes(ctypes.byref(dd), ctypes.byref(pp), M, ctypes.byref(out))
    return st, out.value


def test_workspace_bytes_covers_pool_and_adapt_buffers():
    st, b = _ws(_dict(num_dicts=56, N=4096), _params(), 256)
    assert st == 0
    G = 56 * 256
    assert b >= G * 256 * 6 + G           # pool indices (u16) + pool scores (f32) + status
    st, b2 = _ws(_dict(num_dicts=56, N=4096), _params(), 512)
    assert st == 0 and b2 > b
    st, b0 = _ws(_dict(), _params(), 0)
    assert st == 0


@pytest.mark.parametrize("bad,expect", [
    (dict(d=96), -3), (dict(d=0), -3), (dict(N=0), -3), (dict(N=70000), -3),
    (dict(num_dicts=0), -3), (dict(dtype=7), -2),
])
def test_workspace_rejects_bad_dictionaries(bad, expect):
    st, _ = _ws(_dict(**bad), _params(), 10)
    assert st == expect


@pytest.mark.parametrize("bad,expect", [
    (dict(s=0), -3), (dict(s=33, n=64), -3), (dict(n=4, s=8), -3), (dict(n=513), -3),
    (dict(n=2048), -3), (dict(select=5), -1), (dict(ridge_abs=-1.0), -1),
    (dict(ridge_rel=float("nan")), -1), (dict(delta_key=float("nan")), -1),
    (dict(delta_value=-0.1), -1),
])
def test_workspace_rejects_bad_params(bad, expect):
    st, _ = _ws(_dict(), _params(**bad), 10)
    assert st == expect


def _codes(ptr=FAKE):
    return fadkv.fadkv_codes(ptr, ptr, ptr, ptr)


def _encode(dd, pp, X=FAKE, M=10, codes=None, ws=FAKE, ws_bytes=1 << 40):
    return fadkv.lib().fadkv_encode(ctypes.byref(dd), ctypes.byref(pp), X, M,
                                    ctypes.byref(codes or _codes()), ws, ws_bytes, None)


def test_encode_argument_checks_return_before_any_launch():
    assert _encode(_dict(atoms=None), _params()) == -1
    assert _encode(_dict(atoms=FAKE + 8), _params()) == -1        # atoms not 16-byte aligned
    assert _encode(_dict(), _params(), X=None) == -1
    assert _encode(_dict(), _params(), X=FAKE + 4) == -1
    assert _encode(_dict(), _params(), M=-1) == -1
    assert _encode(_dict(), _params(), codes=fadkv.fadkv_codes(FAKE, None, FAKE, FAKE)) == -1
    assert _encode(_dict(), _params(), codes=fadkv.fadkv_codes(FAKE + 2, FAKE, FAKE, FAKE)) == -1
    assert _encode(_dict(), _params(), ws=None) == -4
    assert _encode(_dict(), _params(), ws_bytes=100) == -4
    assert _encode(_dict(num_dicts=1 << 20), _params(), M=1 << 12) == -3   # >= 2^31 vectors
    assert _encode(_dict(dtype=3), _params()) == -2
    assert _encode(_dict(), _params(n=2000)) == -3


def test_encode_with_no_vectors_is_a_no_op():
    # M = 0: everything checked, nothing launched, no workspace needed
    assert _encode(_dict(), _params(), X=None, M=0, ws=None, ws_bytes=0) == 0


def test_adapt_argument_checks():
    L = fadkv.lib()

    def adapt(dd, pp, X=FAKE, M=10, replaced=FAKE, ws=FAKE, ws_bytes=1 << 40):
        return L.fadkv_adapt(ctypes.byref(dd), ctypes.byref(pp), X, M, ctypes.byref(_codes()),
                             replaced, ws, ws_bytes, None)

    assert adapt(_dict(usage=None), _params()) == -1
    assert adapt(_dict(usage=FAKE + 2), _params()) == -1
    assert adapt(_dict(), _params(), replaced=None) == -1
    assert adapt(_dict(), _params(), ws_bytes=10) == -4
    assert adapt(_dict(), _params(), M=0, X=None, ws=None, ws_bytes=0) == 0


def test_adapt_append_argument_checks():
    L = fadkv.lib()

    def app(dd, pp, X=FAKE, M=10, replaced=FAKE, n_atoms=FAKE, ws=FAKE, ws_bytes=1 << 40):
        return L.fadkv_adapt_append(ctypes.byref(dd), ctypes.byref(pp), X, M,
                                    ctypes.byref(_codes()), replaced, n_atoms, ws, ws_bytes, None)

    assert app(_dict(), _params(), n_atoms=None) == -1
    assert app(_dict(), _params(), n_atoms=FAKE + 2) == -1
    assert app(_dict(usage=None), _params()) == -1
    assert app(_dict(), _params(), replaced=None) == -1
    assert app(_dict(), _params(), X=FAKE + 4) == -1
    assert app(_dict(), _params(), ws_bytes=10) == -4
    assert app(_dict(), _params(s=0)) == -3
    assert app(_dict(), _params(), M=0, X=None, ws=None, ws_bytes=0) == 0


def test_encode_omp_argument_checks():
    L = fadkv.lib()

    def omp(dd, pp, X=FAKE, M=10, ws=FAKE, ws_bytes=1 << 40, codes=None):
        c = _codes() if codes is None else codes
        return L.fadkv_encode_omp(ctypes.byref(dd), ctypes.byref(pp), X, M, ctypes.byref(c), ws,
                                  ws_bytes, None)

    assert omp(_dict(), _params(), X=None) == -1
    assert omp(_dict(), _params(), X=FAKE + 8) == -1
    assert omp(_dict(dtype=7), _params()) == -2
    assert omp(_dict(d=96), _params()) == -3
    assert omp(_dict(N=4), _params(n=8, s=8)) == -3        # s <= n <= N
    assert omp(_dict(), _params(s=33)) == -3
    assert omp(_dict(), _params(), ws_bytes=100) == -4
    assert omp(_dict(), _params(), ws=FAKE + 64) == -4
    assert omp(_dict(), _params(), M=-1) == -1
    assert omp(_dict(), _params(), M=0, X=None, ws=None, ws_bytes=0) == 0
    out = ctypes.c_size_t(0)
    assert L.fadkv_omp_workspace_bytes(ctypes.byref(_dict(num_dicts=56, N=4096)),
                                       ctypes.byref(_params()), 256, ctypes.byref(out)) == 0
    G = 56 * 256
    assert out.value >= G * (1 + 4 + 8 * 4 + 64 * 4 + 8 * 4 + 2 * 128 * 2)
    assert out.value % 256 == 0


def test_reconstruct_argument_checks():
    L = fadkv.lib()

    def rec(dd, idx=FAKE, coef=FAKE, s=8, M=10, out=FAKE, odt=1):
        return L.fadkv_reconstruct(ctypes.byref(dd), idx, coef, s, M, out, odt, None)

    assert rec(_dict(), idx=None) == -1
    assert rec(_dict(), out=FAKE + 8) == -1
    assert rec(_dict(), s=0) == -3
    assert rec(_dict(), s=40) == -3
    assert rec(_dict(), odt=9) == -2
    assert rec(_dict(), M=0) == 0


def test_attend_argument_checks():
    L = fadkv.lib()

    def att(dd, layer=0, s=8, ptrs=FAKE, lens=FAKE, R=16, T=100, q=FAKE, G=3, scale=0.1,
            out=FAKE, ws=FAKE, ws_bytes=1 << 40):
        return L.fadkv_attend(ctypes.byref(dd), layer, s, ptrs, ptrs, ptrs, ptrs, lens, R, T, q,
                              G, scale, out, ws, ws_bytes, None)

    assert att(_dict(num_dicts=2, N=1024), layer=1) == -3           # needs dictionaries 2 and 3
    assert att(_dict(num_dicts=2, N=32768)) == -3                   # N above the LDS budget
    assert att(_dict(), s=0) == -3
    assert att(_dict(), s=33) == -3
    assert att(_dict(), G=0) == -3
    assert att(_dict(), G=65) == -3
    assert att(_dict(), R=-1) == -3
    assert att(_dict(), scale=float("inf")) == -1
    assert att(_dict(), q=FAKE + 4) == -1                           # q must be 16-byte aligned
    assert att(_dict(), lens=None) == -1
    assert att(_dict(), ptrs=None) == -1
    assert att(_dict(), ws_bytes=16) == -4
    assert att(_dict(), ws=FAKE + 16) == -4
    assert att(_dict(), R=0, ptrs=None, lens=None, q=None, out=None, ws=None, ws_bytes=0) == 0


def test_attend_workspace_size():
    L = fadkv.lib()
    out = ctypes.c_size_t(0)
    assert L.fadkv_attend_workspace_bytes(ctypes.byref(_dict(num_dicts=2, N=4096)), 256, 3,
                                          ctypes.byref(out)) == 0
    assert out.value >= 256 * 3 * 4096 * 4 and out.value % 256 == 0
    assert L.fadkv_attend_workspace_bytes(ctypes.byref(_dict(num_dicts=1)), 1, 1,
                                          ctypes.byref(out)) == -3


def test_size_limits_at_the_boundary():
    """The vector-count limit num_dicts * M < 2^31 is accepted right up to the boundary (the
    kernels whose grids grow with it are launched in chunks) and rejected at it; attention takes
    R <= 2^22 rows and R * G <= 2^24 queries, its grids' limits."""
    L = fadkv.lib()
    assert _ws(_dict(num_dicts=2, N=1024), _params(n=64, s=8), (1 << 30) - 1)[0] == 0
    assert _ws(_dict(num_dicts=2, N=1024), _params(n=64, s=8), 1 << 30)[0] == -3
    assert _ws(_dict(num_dicts=1, N=1024), _params(n=512, s=8), (1 << 31) - 1)[0] == 0
    out = ctypes.c_size_t(0)
    ws = lambda R, G: L.fadkv_attend_workspace_bytes(ctypes.byref(_dict(num_dicts=2, N=64)), R, G,
                                                     ctypes.byref(out))
    assert ws(1 << 22, 4) == 0 and ws((1 << 22) + 1, 1) == -3
    assert ws(1 << 18, 64) == 0 and ws(1 << 18, 65) == -3 and ws((1 << 18) + 1, 64) == -3

    def att(R, G):
        return L.fadkv_attend(ctypes.byref(_dict(num_dicts=2, N=64)), 0, 8, FAKE, FAKE, FAKE,
                              FAKE, FAKE, R, 10, FAKE, G, 0.1, FAKE, FAKE, 16, None)
    assert att((1 << 22) + 1, 1) == -3 and att((1 << 18) + 1, 64) == -3
    assert att(1 << 18, 64) == -4        # accepted shape; only the tiny workspace is refused


def test_encode_noalloc_argument_and_scratch_checks():
    """fadkv_encode_noalloc refuses, before touching the GPU, a call whose pools exceed its
    static scratch (FADKV_ERR_SCRATCH) and bad arguments as fadkv_encode does."""
    L = fadkv.lib()
    codes = _codes()

    def enc(dd, pp, M, X=FAKE):
        return L.fadkv_encode_noalloc(ctypes.byref(dd), ctypes.byref(pp), X, M,
                                      ctypes.byref(codes), None)
    dd, pp = _dict(num_dicts=56, N=4096), _params()
    st, need = _ws(dd, pp, 256)
    assert st == 0 and need <= fadkv.NOALLOC_SCRATCH_BYTES      # the 3B decode step fits
    assert enc(dd, pp, 2000) == fadkv.FADKV_ERR_SCRATCH
    assert enc(dd, pp, 10, X=FAKE + 8) == -1
    assert enc(_dict(d=96), pp, 10) == -3
    assert enc(dd, _params(n=4), 10) == -3
    assert enc(dd, pp, 0) == 0
    assert fadkv.fadkv_status_string(fadkv.FADKV_ERR_SCRATCH) != "unknown status"
