"""Pins for the oracle's chunked / variable-length prefill against a cache and
its sliding window (CPU only).

Reading of the window (the pages pass a ``sliding_window`` to the flash
attention call of "llama.py — LLaMA 注意力层 Ulysses SP 适配", section
"第二步：RoPE + Flash Attention", without defining it): a query at absolute
position p sees keys p - W < j <= p.  The pins below check the oracle against
scalar loops written from that sentence, against torch's CPU float64
scaled_dot_product_attention given a band mask built with torch's own
tril/triu, and against closed forms and the plain prefill / decode oracles.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _qkv(seed, B, Sq, Sk, Hq, Hkv, D):
    r = _rng(seed)
    return (r.standard_normal((B, Sq, Hq, D)), r.standard_normal((B, Sk, Hkv, D)),
            r.standard_normal((B, Sk, Hkv, D)))


def _brute_window(q, k, v, scale, window):
    """Scalar loops: query i at position p = i + Sk - Sq sees p - W < j <= p."""
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    out = np.zeros(q.shape)
    for b in range(B):
        for h in range(Hq):
            for i in range(Sq):
                p = i + Sk - Sq
                keys = [j for j in range(Sk) if j <= p and (window == 0 or j > p - window)]
                if not keys:
                    continue
                sc = [scale * sum(float(q[b, i, h, d]) * float(k[b, j, h // G, d]) for d in range(D)) for j in keys]
                mx = max(sc)
                e = [math.exp(x - mx) for x in sc]
                tot = sum(e)
                for d in range(D):
                    out[b, i, h, d] = sum(e[t] * float(v[b, j, h // G, d]) for t, j in enumerate(keys)) / tot
    return out


def _to_cache(k, max_kv):
    """[B,S,Hkv,D] -> [B,Hkv,max_kv,D], rows past S filled with large junk."""
    B, S, Hkv, D = k.shape
    c = np.full((B, Hkv, max_kv, D), 1e3)
    c[:, :, :S] = np.transpose(k, (0, 2, 1, 3))
    return c


@pytest.mark.parametrize("B,Sq,Sk,Hq,Hkv,D,W", [
    (1, 6, 6, 2, 1, 4, 1), (1, 6, 6, 2, 1, 4, 3), (2, 9, 9, 4, 2, 3, 4), (1, 4, 9, 2, 2, 5, 2),
    (1, 1, 7, 4, 1, 4, 3), (1, 5, 5, 2, 1, 2, 0), (2, 7, 7, 2, 1, 4, 50)])
def test_window_brute_force(B, Sq, Sk, Hq, Hkv, D, W):
    q, k, v = _qkv(B + Sq * 10 + Sk * 100 + W, B, Sq, Sk, Hq, Hkv, D)
    np.testing.assert_allclose(oracle.attention(q, k, v, True, 0.6, window=W), _brute_window(q, k, v, 0.6, W),
                               rtol=0, atol=1e-12)


@pytest.mark.parametrize("S,W", [(33, 5), (64, 16), (17, 1)])
def test_window_matches_torch_sdpa_band_mask(S, W):
    q, k, v = _qkv(S * 3 + W, 2, S, S, 4, 2, 16)
    G = 2
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).permute(0, 2, 1, 3)
    ones = torch.ones(S, S, dtype=torch.bool)
    band = ones.tril(0) & ones.triu(-(W - 1))        # keep i - W < j <= i
    ref = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(np.repeat(k, G, axis=2)), t(np.repeat(v, G, axis=2)), attn_mask=band, scale=0.3)
    np.testing.assert_allclose(oracle.attention(q, k, v, True, 0.3, window=W), ref.permute(0, 2, 1, 3).numpy(),
                               rtol=0, atol=1e-12)


def test_window_special_cases():
    q, k, v = _qkv(5, 2, 12, 12, 4, 2, 8)
    full = oracle.attention(q, k, v, True, 0.5)
    # a window at least as long as the sequence changes nothing
    np.testing.assert_allclose(oracle.attention(q, k, v, True, 0.5, window=12), full, rtol=0, atol=0)
    # window 1: each query sees only its own key, so the output is its own value row
    one = oracle.attention(q, k, v, True, 0.5, window=1)
    np.testing.assert_allclose(one, np.repeat(v, 2, axis=2), rtol=0, atol=1e-15)
    with pytest.raises(ValueError):
        oracle.attention(q, k, v, False, 0.5, window=3)


def test_window_int32_max_is_no_window():
    """A window of 2^31 - 1 keys excludes nothing, also for a chunk longer than
    the cache (rows before the first key stay zero rows)."""
    B, Sq, Hq, Hkv, D, max_kv = 2, 12, 4, 2, 8, 9
    q, k, v = _qkv(33, B, Sq, max_kv, Hq, Hkv, D)
    kc, vc = _to_cache(k, max_kv), _to_cache(v, max_kv)
    lens = np.array([5, 9])
    big = oracle.attention_cache(q, kc, vc, lens, True, 0.4, window=2 ** 31 - 1)
    none = oracle.attention_cache(q, kc, vc, lens, True, 0.4, window=0)
    np.testing.assert_array_equal(big, none)
    assert np.all(big[0, :Sq - 5] == 0.0)


@pytest.mark.parametrize("W", [0, 5])
def test_cache_full_chunk_equals_prefill(W):
    B, S, Hq, Hkv, D, max_kv = 2, 20, 4, 2, 8, 31
    q, k, v = _qkv(21, B, S, S, Hq, Hkv, D)
    got = oracle.attention_cache(q, _to_cache(k, max_kv), _to_cache(v, max_kv), np.full(B, S), True, 0.4, window=W)
    np.testing.assert_allclose(got, oracle.attention(q, k, v, True, 0.4, window=W), rtol=0, atol=1e-12)


def test_cache_single_query_equals_decode():
    B, S, Hq, Hkv, D, max_kv = 3, 25, 8, 2, 8, 30
    q, k, v = _qkv(22, B, S, S, Hq, Hkv, D)
    lens = np.array([1, 13, 25])
    kc, vc = _to_cache(k, max_kv), _to_cache(v, max_kv)
    qd = q[np.arange(B), lens - 1]                                     # [B,Hq,D]
    got = oracle.attention_cache(qd[:, None], kc, vc, lens, True, 0.7)[:, 0]
    np.testing.assert_allclose(got, oracle.decode(qd, kc, vc, lens, 0.7), rtol=0, atol=1e-12)


@pytest.mark.parametrize("W", [0, 7])
def test_chunked_prefill_equals_full_prefill(W):
    # feeding a sequence in chunks against the growing cache reproduces the
    # rows of the one-shot prefill
    B, n, Hq, Hkv, D, max_kv = 2, 40, 4, 1, 8, 48
    q, k, v = _qkv(23, B, n, n, Hq, Hkv, D)
    full = oracle.attention(q, k, v, True, 0.35, window=W)
    kc, vc = _to_cache(k, max_kv), _to_cache(v, max_kv)
    for c0, c1 in [(0, 9), (9, 10), (10, 33), (33, 40)]:
        part = oracle.attention_cache(q[:, c0:c1], kc, vc, np.full(B, c1), True, 0.35, window=W)
        np.testing.assert_allclose(part, full[:, c0:c1], rtol=0, atol=1e-12)


def test_cache_variable_lengths_and_degenerate_rows():
    B, Sq, Hq, Hkv, D, max_kv = 4, 6, 2, 1, 4, 9
    r = _rng(24)
    q = r.standard_normal((B, Sq, Hq, D))
    kc, vc = r.standard_normal((B, Hkv, max_kv, D)), r.standard_normal((B, Hkv, max_kv, D))
    lens = np.array([0, 3, 6, 99])                    # 99 is clamped to max_kv
    got = oracle.attention_cache(q, kc, vc, lens, True, 1.0)
    assert np.all(got[0] == 0.0)                      # empty cache: zero rows
    neg = oracle.attention_cache(q, kc, vc, np.array([-4, 3, 6, 99]), True, 1.0)
    assert np.all(neg[0] == 0.0)                      # a negative length is an empty cache
    assert np.all(got[1, :3] == 0.0)                  # queries before the first key see nothing
    for b, L in [(1, 3), (2, 6), (3, max_kv)]:
        n = min(Sq, L)
        kk = np.transpose(kc[b:b + 1, :, :L], (0, 2, 1, 3))
        vv = np.transpose(vc[b:b + 1, :, :L], (0, 2, 1, 3))
        ref = oracle.attention(q[b:b + 1, Sq - n:], kk, vv, True, 1.0)
        np.testing.assert_allclose(got[b, Sq - n:], ref[0], rtol=0, atol=1e-12)
    # non-causal: every query sees all kv_len keys
    nc = oracle.attention_cache(q, kc, vc, lens, False, 1.0)
    kk = np.transpose(kc[2:3, :, :6], (0, 2, 1, 3))
    vv = np.transpose(vc[2:3, :, :6], (0, 2, 1, 3))
    np.testing.assert_allclose(nc[2], oracle.attention(q[2:3], kk, vv, False, 1.0)[0], rtol=0, atol=1e-12)
