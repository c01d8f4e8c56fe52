"""Pins of the attention oracle (CPU only): a library attention routine, closed forms and
invariances, each chosen so that a dropped scale, a missing max shift, a transposed
key/value or an off-by-one token count fails one of them."""
import numpy as np
import pytest
import torch

from oracle import attend_oracle as ao


def _case(rng, R=3, T=7, s=3, G=2, N=20, d=8):
    Dk = rng.standard_normal((N, d))
    Dv = rng.standard_normal((N, d))
    k_idx = rng.integers(0, N, (R, T, s)).astype(np.int32)
    v_idx = rng.integers(0, N, (R, T, s)).astype(np.int32)
    k_coef = rng.standard_normal((R, T, s)).astype(np.float32)
    v_coef = rng.standard_normal((R, T, s)).astype(np.float32)
    q = rng.standard_normal((R, G, d))
    return Dk, Dv, k_idx, k_coef, v_idx, v_coef, q


def test_matches_torch_sdpa_on_rebuilt_tokens():
    rng = np.random.default_rng(1)
    Dk, Dv, ki, kc, vi, vc, q = _case(rng)
    lens = np.array([7, 4, 1])
    scale = 0.37
    out = ao.attend(Dk, Dv, ki, kc, vi, vc, lens, q, scale)
    for r in range(3):
        L = lens[r]
        K = torch.zeros(L, Dk.shape[1], dtype=torch.float64)
        V = torch.zeros(L, Dv.shape[1], dtype=torch.float64)
        for t in range(L):
            for k in range(ki.shape[2]):
                K[t] += float(kc[r, t, k]) * torch.from_numpy(Dk[ki[r, t, k]])
                V[t] += float(vc[r, t, k]) * torch.from_numpy(Dv[vi[r, t, k]])
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[r])[None], K[None], V[None], scale=scale)[0]
        np.testing.assert_allclose(out[r], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_single_token_returns_its_value():
    rng = np.random.default_rng(2)
    Dk, Dv, ki, kc, vi, vc, q = _case(rng, R=1, T=1)
    out = ao.attend(Dk, Dv, ki, kc, vi, vc, np.array([1]), q, 3.0)
    v0 = sum(float(vc[0, 0, k]) * Dv[vi[0, 0, k]] for k in range(vc.shape[2]))
    np.testing.assert_allclose(out[0, 0], v0, rtol=1e-13)
    np.testing.assert_allclose(out[0, 1], v0, rtol=1e-13)


def test_zero_query_averages_values():
    rng = np.random.default_rng(3)
    Dk, Dv, ki, kc, vi, vc, q = _case(rng, R=1, T=5)
    q[:] = 0.0
    out = ao.attend(Dk, Dv, ki, kc, vi, vc, np.array([5]), q, 1.0)
    V = ao.rebuild(Dv, vi[0], vc[0])
    np.testing.assert_allclose(out[0, 0], V.mean(axis=0), rtol=1e-13)


def test_two_token_hand_example():
    # keys e0 and log(3) e0 under q = e0, scale 1: logits 0 and log 3, p = (1/4, 3/4)
    Dk = np.eye(2)
    Dv = np.array([[4.0, 0.0], [0.0, 8.0]])
    ki = np.array([[[0], [0]]], np.int32)
    kc = np.array([[[0.0], [np.log(3.0)]]])
    vi = np.array([[[0], [1]]], np.int32)
    vc = np.ones((1, 2, 1))
    q = np.array([[[1.0, 0.0]]])
    out = ao.attend(Dk, Dv, ki, kc, vi, vc, np.array([2]), q, 1.0)
    np.testing.assert_allclose(out[0, 0], [1.0, 6.0], rtol=1e-14)


def test_token_order_and_empty_slots():
    rng = np.random.default_rng(4)
    Dk, Dv, ki, kc, vi, vc, q = _case(rng, R=1, T=6)
    base = ao.attend(Dk, Dv, ki, kc, vi, vc, np.array([6]), q, 0.5)
    perm = rng.permutation(6)
    out = ao.attend(Dk, Dv, ki[:, perm], kc[:, perm], vi[:, perm], vc[:, perm], np.array([6]), q, 0.5)
    np.testing.assert_allclose(out, base, rtol=1e-12)
    # an extra empty slot (idx -1, any coefficient) changes nothing
    ki2 = np.concatenate([ki, -np.ones((1, 6, 1), np.int32)], axis=2)
    kc2 = np.concatenate([kc, 9.0 * np.ones((1, 6, 1), np.float32)], axis=2)
    vi2 = np.concatenate([vi, -np.ones((1, 6, 1), np.int32)], axis=2)
    vc2 = np.concatenate([vc, 9.0 * np.ones((1, 6, 1), np.float32)], axis=2)
    np.testing.assert_allclose(ao.attend(Dk, Dv, ki2, kc2, vi2, vc2, np.array([6]), q, 0.5), base,
                               rtol=1e-13)


def test_tokens_past_len_and_empty_rows_are_ignored():
    rng = np.random.default_rng(5)
    Dk, Dv, ki, kc, vi, vc, q = _case(rng, R=2, T=6)
    out = ao.attend(Dk, Dv, ki, kc, vi, vc, np.array([3, 0]), q, 0.5)
    short = ao.attend(Dk, Dv, ki[:, :3], kc[:, :3], vi[:, :3], vc[:, :3], np.array([3, 0]), q, 0.5)
    np.testing.assert_allclose(out, short, rtol=1e-14)
    assert np.all(out[1] == 0.0)


@pytest.mark.parametrize("shift", [0.0, 800.0])
def test_softmax_is_shift_invariant_and_overflow_safe(shift):
    # adding the same amount to every logit (via a key component along q) changes nothing,
    # and large logits do not overflow
    Dk = np.array([[1.0, 0.0], [0.0, 1.0]])
    Dv = np.array([[1.0, 2.0], [3.0, -1.0]])
    ki = np.array([[[0, 1], [0, 1]]], np.int32)
    kc = np.array([[[shift, 0.5], [shift, -0.5]]])
    vi = np.array([[[0, 0], [1, 1]]], np.int32)
    vc = np.array([[[1.0, 0.0], [1.0, 0.0]]])
    q = np.array([[[1.0, 1.0]]])
    out = ao.attend(Dk, Dv, ki, kc, vi, vc, np.array([2]), q, 1.0)
    p0 = 1.0 / (1.0 + np.exp(-1.0))
    np.testing.assert_allclose(out[0, 0], p0 * Dv[0] + (1 - p0) * Dv[1], rtol=1e-12)
