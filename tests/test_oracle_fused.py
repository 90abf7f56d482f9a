"""Pins for the oracle's rotation-then-attention steps (CPU only).

Each pin ties the composed function to a property the pages and the
mathematics fix, not to a retyping of the composition:

* RoPE encodes relative position ("LLaMA2大语言模型架构详解", section "Rotary
  Position Encoding"): shifting every position of a sequence by the same t
  leaves every score, hence the attention output, unchanged.  Rotating only q
  or only k, rotating v, or giving q and k different positions breaks it.
* Position 0 is no rotation: the result is plain attention.
* Linear scaling divides positions ("Llama2 Transformer架构解析与优化实践",
  section 6.1): positions 2p with factor 2 equal positions p with factor 1.
* A decode step after appending the new token to the cache ("LLaMA2大语言模型
  架构详解", section "KV cache") gives the same row as causal prefill of the
  whole sequence -- fed token by token, the cache reproduces every prefill row.
"""
import numpy as np
import pytest

import oracle


def _qkv(seed, B, S, Hq, Hkv, D):
    r = np.random.Generator(np.random.PCG64(seed))
    return (r.standard_normal((B, S, Hq, D)), r.standard_normal((B, S, Hkv, D)),
            r.standard_normal((B, S, Hkv, D)))


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shift", [1, 37, 1000])
def test_shift_invariance(causal, shift):
    q, k, v = _qkv(3 + shift, 2, 11, 4, 2, 8)
    pos = np.broadcast_to(np.arange(11), (2, 11))
    a, _ = oracle.rope_attention(q, k, v, pos, causal, 0.4, 10000.0)
    b, _ = oracle.rope_attention(q, k, v, pos + shift, causal, 0.4, 10000.0)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-10)


def test_shift_invariance_catches_one_sided_rotation():
    # the property is not vacuous: rotating the queries alone breaks it
    q, k, v = _qkv(4, 1, 9, 2, 1, 8)
    pos = np.broadcast_to(np.arange(9), (1, 9))

    def q_only(p):
        q_rot = oracle.rotate(q, p[:, :, None], 10000.0)
        return oracle.attention(q_rot, k, v, True, 0.5)
    assert np.abs(q_only(pos) - q_only(pos + 5)).max() > 1e-3


def test_zero_positions_is_plain_attention():
    q, k, v = _qkv(5, 2, 10, 4, 2, 8)
    out, k_rot = oracle.rope_attention(q, k, v, np.zeros((2, 10), dtype=int), True, 0.3, 10000.0)
    np.testing.assert_array_equal(out, oracle.attention(q, k, v, True, 0.3))
    np.testing.assert_array_equal(k_rot, k)


def test_linear_factor_scales_positions():
    q, k, v = _qkv(6, 1, 12, 2, 2, 8)
    pos = np.broadcast_to(np.arange(12), (1, 12))
    a, _ = oracle.rope_attention(q, k, v, 2 * pos, True, 0.3, 500.0, linear_factor=2.0)
    b, _ = oracle.rope_attention(q, k, v, pos, True, 0.3, 500.0)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


@pytest.mark.parametrize("factor", [1.0, 2.0])
def test_decode_steps_reproduce_prefill_rows(factor):
    B, n, Hq, Hkv, D, max_kv = 2, 9, 4, 2, 8, 12
    q, k, v = _qkv(7, B, n, Hq, Hkv, D)
    full, k_rot = oracle.rope_attention(q, k, v, None, True, 0.35, 10000.0, factor)
    kc = np.full((B, Hkv, max_kv, D), 7.0)      # junk beyond the filled rows
    vc = np.full((B, Hkv, max_kv, D), -7.0)
    for t in range(n):
        lens = np.full(B, t + 1)
        out, kc, vc = oracle.rope_decode_step(q[:, t], k[:, t], v[:, t], kc, vc, lens, None, 0.35, 10000.0,
                                              factor)
        np.testing.assert_allclose(out, full[:, t], rtol=0, atol=1e-12)
    # the cache holds the rotated keys of the prefill and the raw values
    np.testing.assert_allclose(kc[:, :, :n], np.transpose(k_rot, (0, 2, 1, 3)), rtol=0, atol=1e-13)
    np.testing.assert_array_equal(vc[:, :, :n], np.transpose(v, (0, 2, 1, 3)))


def test_decode_step_explicit_positions_and_skipped_rows():
    B, Hq, Hkv, D, max_kv = 3, 4, 1, 8, 6
    r = np.random.Generator(np.random.PCG64(8))
    q, kn, vn = r.standard_normal((B, Hq, D)), r.standard_normal((B, Hkv, D)), r.standard_normal((B, Hkv, D))
    kc, vc = r.standard_normal((B, Hkv, max_kv, D)), r.standard_normal((B, Hkv, max_kv, D))
    lens = np.array([3, 0, 9])                   # row 2; no row; row 8 is outside the cache
    out, kc2, vc2 = oracle.rope_decode_step(q, kn, vn, kc, vc, lens, np.array([40, 5, 7]), 0.5, 10000.0)
    np.testing.assert_allclose(kc2[0, :, 2], oracle.rotate(kn[0], 40, 10000.0), rtol=0, atol=0)
    np.testing.assert_array_equal(kc2[1:], kc[1:])   # nothing written for rows -1 and 8
    np.testing.assert_array_equal(out[1], 0.0)       # empty cache: zero row
    # moving the new token alone turns its query against the cached keys
    out_b, _, _ = oracle.rope_decode_step(q, kn, vn, kc, vc, lens, np.array([41, 5, 7]), 0.5, 10000.0)
    assert np.abs(out_b[0] - out[0]).max() > 1e-6
