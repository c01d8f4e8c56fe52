"""fadkv_encode_noalloc (the encode entry point for callers that cannot allocate) against
fadkv_encode through the C ABI: two calls in a row on one GPU, the second with a smaller input
than the first, must give the same codes bit for bit as fadkv_encode with its own workspace
(the same kernels run on the same inputs; only the scratch differs).  A call larger than the
static scratch is refused before anything is launched."""
import numpy as np
import pytest
import torch

from sparse_dictionary_coding_amd import fadkv, synth
from sparse_dictionary_coding_amd.synth import SyntheticKV

from . import parity

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _same(a: fadkv.Codes, b: fadkv.Codes):
    for u, v in zip(parity.codes_to_numpy(a), parity.codes_to_numpy(b)):
        np.testing.assert_array_equal(u, v)


def test_noalloc_encode_matches_encode_twice_second_smaller():
    w = synth.WORKLOADS["llama3b_decode"]
    g = SyntheticKV(w, device=DEV)
    A = g.atoms()
    p = fadkv.Params(n=w.n, s=w.s)
    X1 = g.batch(A, step=0)                                  # 56 x 256 vectors (22 MB of pools)
    X2 = g.batch(A, step=1)[:, :37].contiguous()             # 56 x 37: a smaller second call
    print(f"[no-alloc] call 1: {tuple(X1.shape)}, call 2: {tuple(X2.shape)}", flush=True)
    got1 = fadkv.fadkv_encode_noalloc(A, X1, p)
    got2 = fadkv.fadkv_encode_noalloc(A, X2, p)
    torch.cuda.synchronize()
    ref1 = fadkv.fadkv_encode(A, X1, p)
    ref2 = fadkv.fadkv_encode(A, X2, p)
    torch.cuda.synchronize()
    _same(got1, ref1)
    _same(got2, ref2)
    # the same again with PL and a different dictionary shape (8B decode: n = 512, s = 16)
    w8 = synth.WORKLOADS["llama8b_decode"]
    g8 = SyntheticKV(w8, device=DEV, num_dicts=16)
    A8 = g8.atoms()
    for select in ("pl", "gm"):
        p8 = fadkv.Params(n=w8.n, s=w8.s, select=select)
        X8 = g8.batch(A8, step=2)
        got = fadkv.fadkv_encode_noalloc(A8, X8, p8)
        got_small = fadkv.fadkv_encode_noalloc(A8, X8[:, :5].contiguous(), p8)
        torch.cuda.synchronize()
        _same(got, fadkv.fadkv_encode(A8, X8, p8))
        _same(got_small, fadkv.fadkv_encode(A8, X8[:, :5].contiguous(), p8))
    torch.cuda.synchronize()


def test_noalloc_refuses_calls_beyond_its_scratch():
    w = synth.WORKLOADS["llama3b_decode"]
    g = SyntheticKV(w, device=DEV, num_dicts=2)
    A = g.atoms()
    p = fadkv.Params(n=w.n, s=w.s)
    M = fadkv.NOALLOC_SCRATCH_BYTES // (2 * (6 * w.n + 1)) + 64      # just over the scratch
    X = torch.zeros(2, M, w.d, dtype=A.dtype, device=DEV)
    with pytest.raises(fadkv.FadkvError) as e:
        fadkv.fadkv_encode_noalloc(A, X, p)
    assert e.value.status == fadkv.FADKV_ERR_SCRATCH
