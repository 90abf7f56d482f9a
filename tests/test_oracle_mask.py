"""Pins of the oracle's general additive mask (oracle.attention(mask=...)):
a zero mask changes nothing, a -inf upper triangle is the causal mask, a
per-row constant shifts nothing (softmax invariance), -inf on trailing keys
equals attention over the shorter key range, a per-head mask equal for all
heads equals the shared one, fully masked rows are zeros, and a tiny case by
explicit loops."""
import math

import numpy as np
import pytest

import oracle


def _qkv(seed, B=2, S=9, Hq=4, Hkv=2, D=8, Sk=None):
    rng = np.random.Generator(np.random.PCG64(seed))
    Sk = S if Sk is None else Sk
    return (rng.standard_normal((B, S, Hq, D)), rng.standard_normal((B, Sk, Hkv, D)),
            rng.standard_normal((B, Sk, Hkv, D)))


def test_zero_mask_is_identity():
    q, k, v = _qkv(1)
    for causal in (False, True):
        a = oracle.attention(q, k, v, causal, 0.3)
        b = oracle.attention(q, k, v, causal, 0.3, mask=np.zeros((2, 1, 9, 9)))
        assert np.array_equal(a, b)


def test_upper_triangle_is_causal():
    q, k, v = _qkv(2)
    tri = np.where(np.arange(9)[None, :] > np.arange(9)[:, None], -np.inf, 0.0)
    m = np.broadcast_to(tri, (2, 1, 9, 9))
    assert np.array_equal(oracle.attention(q, k, v, False, 0.3, mask=m), oracle.attention(q, k, v, True, 0.3))


def test_row_shift_invariance():
    q, k, v = _qkv(3)
    rng = np.random.Generator(np.random.PCG64(3))
    m = rng.standard_normal((2, 4, 9, 9))
    shift = rng.standard_normal((2, 4, 9, 1)) * 50
    a = oracle.attention(q, k, v, True, 0.3, mask=m)
    b = oracle.attention(q, k, v, True, 0.3, mask=m + shift)
    np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)


def test_key_padding_equals_shorter_keys():
    q, k, v = _qkv(4)
    L = 6
    m = np.zeros((2, 1, 9, 9))
    m[:, :, :, L:] = -np.inf
    a = oracle.attention(q, k, v, False, 0.3, mask=m)
    b = oracle.attention(q, k[:, :L], v[:, :L], False, 0.3)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)


def test_per_head_mask_equal_to_shared():
    q, k, v = _qkv(5)
    m1 = np.random.Generator(np.random.PCG64(5)).standard_normal((2, 1, 9, 9))
    mh = np.repeat(m1, 4, axis=1)
    assert np.array_equal(oracle.attention(q, k, v, True, 0.3, mask=m1), oracle.attention(q, k, v, True, 0.3, mask=mh))


def test_fully_masked_rows_are_zero():
    q, k, v = _qkv(6)
    m = np.zeros((2, 1, 9, 9))
    m[0, 0, 3, :] = -np.inf
    out = oracle.attention(q, k, v, False, 0.3, mask=m)
    assert np.all(out[0, 3] == 0.0) and np.all(np.isfinite(out))


def test_tiny_case_by_loops():
    q, k, v = _qkv(7, B=1, S=3, Hq=2, Hkv=1, D=4)
    m = np.random.Generator(np.random.PCG64(7)).standard_normal((1, 2, 3, 3))
    out = oracle.attention(q, k, v, True, 0.5, mask=m)
    for h in range(2):
        for i in range(3):
            w = [math.exp(0.5 * sum(q[0, i, h, d] * k[0, j, 0, d] for d in range(4)) + m[0, h, i, j]) if j <= i else 0.0
                 for j in range(3)]
            ref = [sum(w[j] * v[0, j, 0, d] for j in range(3)) / sum(w) for d in range(4)]
            np.testing.assert_allclose(out[0, i, h], ref, rtol=1e-12)


def test_rejects_bad_mask_shape():
    q, k, v = _qkv(8)
    with pytest.raises(ValueError):
        oracle.attention(q, k, v, True, 0.3, mask=np.zeros((2, 3, 9, 9)))
