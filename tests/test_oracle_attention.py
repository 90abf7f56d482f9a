"""Pins for the attention oracle (CPU only).

Checks against: torch's CPU scaled_dot_product_attention in float64 (the
library routine one of the pages' attention variants calls), brute-force
scalar loops on tiny shapes, closed forms (uniform scores give prefix means,
one key returns its value), invariants (rows sum to one, masked weights are
zero, GQA equals MHA on repeated K/V, decode equals the last prefill row) and
the hand fixtures under tests/golden.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from tests.conftest import GOLDEN


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _qkv(seed, B, Sq, Sk, Hq, Hkv, D):
    r = _rng(seed)
    return (r.standard_normal((B, Sq, Hq, D)), r.standard_normal((B, Sk, Hkv, D)),
            r.standard_normal((B, Sk, Hkv, D)))


def _brute(q, k, v, causal, scale):
    """Scalar loops, math.exp, no numpy arithmetic."""
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    out = np.zeros(q.shape)
    for b in range(B):
        for h in range(Hq):
            kh = h // G
            for i in range(Sq):
                keys = [j for j in range(Sk) if not (causal and j > i + Sk - Sq)]
                sc = []
                for j in keys:
                    acc = 0.0
                    for d in range(D):
                        acc += float(q[b, i, h, d]) * float(k[b, j, kh, d])
                    sc.append(scale * acc)
                if not sc:
                    continue
                mx = max(sc)
                e = [math.exp(x - mx) for x in sc]
                tot = sum(e)
                for d in range(D):
                    out[b, i, h, d] = sum(e[t] * float(v[b, j, kh, d]) for t, j in enumerate(keys)) / tot
    return out


def _sdpa(q, k, v, causal, scale=None):
    """torch CPU float64 SDPA on [B,S,H,D] inputs with K/V repeated per group."""
    G = q.shape[2] // k.shape[2]
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).permute(0, 2, 1, 3)
    kk = t(np.repeat(k, G, axis=2))
    vv = t(np.repeat(v, G, axis=2))
    o = torch.nn.functional.scaled_dot_product_attention(t(q), kk, vv, is_causal=causal, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


SHAPES = [(B, S, Hq, Hkv, D, c)
          for (B, S, Hq, Hkv, D, c) in itertools.product([1, 2], [1, 2, 5, 9], [1, 2, 4], [1, 2], [2, 4, 8], [False, True])
          if Hq % Hkv == 0]


@pytest.mark.parametrize("B,S,Hq,Hkv,D,causal", SHAPES)
def test_brute_force_tiny(B, S, Hq, Hkv, D, causal):
    q, k, v = _qkv(B * 1000 + S * 100 + Hq * 10 + Hkv + D, B, S, S, Hq, Hkv, D)
    scale = 0.37
    np.testing.assert_allclose(oracle.attention(q, k, v, causal, scale), _brute(q, k, v, causal, scale),
                               rtol=0, atol=1e-12)


@pytest.mark.parametrize("B,Sq,Sk,Hq,Hkv,D", [(1, 3, 7, 2, 1, 4), (2, 1, 6, 4, 2, 8), (1, 5, 5, 4, 4, 2)])
def test_brute_force_bottom_right(B, Sq, Sk, Hq, Hkv, D):
    q, k, v = _qkv(77, B, Sq, Sk, Hq, Hkv, D)
    np.testing.assert_allclose(oracle.attention(q, k, v, True, 0.5), _brute(q, k, v, True, 0.5), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,S,Hq,Hkv,D", [(2, 33, 8, 2, 64), (1, 130, 4, 1, 128), (2, 17, 6, 3, 32)])
def test_matches_torch_sdpa_fp64(B, S, Hq, Hkv, D, causal):
    q, k, v = _qkv(S + D, B, S, S, Hq, Hkv, D)
    # scale=None: SDPA's own default 1/sqrt(D) -- pins the scale convention too
    np.testing.assert_allclose(oracle.attention(q, k, v, causal, 1.0 / math.sqrt(D)), _sdpa(q, k, v, causal),
                               rtol=0, atol=1e-12)
    np.testing.assert_allclose(oracle.attention(q, k, v, causal, 0.2), _sdpa(q, k, v, causal, 0.2),
                               rtol=0, atol=1e-12)


def test_rows_sum_to_one_and_masked_are_zero():
    q, k, _ = _qkv(11, 1, 40, 40, 4, 2, 16)
    for h in range(4):
        p = oracle.attention_probs(q, k, 0.25, True, 0, h)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        iu = np.triu_indices(40, 1)
        assert np.all(p[iu] == 0.0)
        assert np.all(p[np.tril_indices(40)] > 0.0)
        pu = oracle.attention_probs(q, k, 0.25, False, 0, h)
        assert np.all(pu > 0.0)


def test_gqa_equals_mha_on_repeated_kv():
    q, k, v = _qkv(12, 2, 19, 19, 8, 2, 16)
    G = 4
    for causal in (False, True):
        a = oracle.attention(q, k, v, causal, 0.3)
        b = oracle.attention(q, np.repeat(k, G, axis=2), np.repeat(v, G, axis=2), causal, 0.3)
        np.testing.assert_array_equal(a, b)


def test_head_map_fixture():
    g = json.load(open(os.path.join(GOLDEN, "gqa_head_map.json")))
    Hq, Hkv = g["Hq"], g["Hkv"]
    q, k, _ = _qkv(13, 1, 3, 3, Hq, Hkv, 4)
    v = np.zeros((1, 3, Hkv, 4))
    for kh in range(Hkv):
        v[:, :, kh, :] = kh          # a value that names its K/V head
    out = oracle.attention(q, k, v, True, 0.5)
    np.testing.assert_allclose(out[0, :, :, 0], np.tile(np.array(g["kv_head_of_query_head"], float), (3, 1)),
                               rtol=0, atol=1e-12)


def test_single_key_returns_value():
    q, k, v = _qkv(14, 2, 1, 1, 4, 2, 8)
    out = oracle.attention(q, k, v, True, 1.0)
    np.testing.assert_array_equal(out, np.repeat(v, 2, axis=2))
    dq = q[:, 0]
    kc, vc = np.transpose(k, (0, 2, 1, 3)), np.transpose(v, (0, 2, 1, 3))
    np.testing.assert_array_equal(oracle.decode(dq, kc, vc, np.array([1, 1]), 1.0), np.repeat(v[:, 0], 2, axis=1))


def test_uniform_scores_give_prefix_means():
    _, k, v = _qkv(15, 1, 12, 12, 2, 1, 8)
    q = np.zeros((1, 12, 2, 8))
    out = oracle.attention(q, k, v, True, 1.0)
    for i in range(12):
        np.testing.assert_allclose(out[0, i, 1], v[0, : i + 1, 0].mean(axis=0), rtol=0, atol=1e-14)
    out = oracle.attention(q, k, v, False, 1.0)
    np.testing.assert_allclose(out[0, :, 0], np.broadcast_to(v[0, :, 0].mean(axis=0), (12, 8)), rtol=0, atol=1e-14)


def test_decode_equals_last_prefill_row():
    B, n, Hq, Hkv, D, max_kv = 3, 23, 8, 2, 16, 40
    q, k, v = _qkv(16, B, n, n, Hq, Hkv, D)
    full = oracle.attention(q, k, v, True, 0.25)
    kc = np.zeros((B, Hkv, max_kv, D))
    vc = np.zeros((B, Hkv, max_kv, D))
    kc[:, :, :n] = np.transpose(k, (0, 2, 1, 3))
    vc[:, :, :n] = np.transpose(v, (0, 2, 1, 3))
    kc[:, :, n:] = 1e3          # rows past kv_len must not matter
    dec = oracle.decode(q[:, -1], kc, vc, np.full(B, n), 0.25)
    np.testing.assert_allclose(dec, full[:, -1], rtol=0, atol=1e-12)
    # per-sequence lengths: sequence b uses its own prefix
    lens = np.array([1, 7, n])
    dec = oracle.decode(q[np.arange(B), lens - 1], kc, vc, lens, 0.25)
    for b, L in enumerate(lens):
        ref = oracle.attention(q[b:b + 1, L - 1:L], k[b:b + 1, :L], v[b:b + 1, :L], True, 0.25)
        np.testing.assert_allclose(dec[b], ref[0, 0], rtol=0, atol=1e-12)


def test_decode_lengths_are_clamped():
    B, Hq, Hkv, D, max_kv = 2, 2, 1, 4, 5
    r = _rng(17)
    q = r.standard_normal((B, Hq, D))
    kc, vc = r.standard_normal((B, Hkv, max_kv, D)), r.standard_normal((B, Hkv, max_kv, D))
    out = oracle.decode(q, kc, vc, np.array([0, 99]), 1.0)
    assert np.all(out[0] == 0.0)
    assert np.all(oracle.decode(q, kc, vc, np.array([-3, 99]), 1.0)[0] == 0.0)   # negative: no keys
    np.testing.assert_array_equal(out[1], oracle.decode(q, kc, vc, np.array([0, max_kv]), 1.0)[1])


def test_chunk_of_queries_equals_tail_of_full_prefill():
    # bottom-right alignment: the last Sq queries against all Sk keys are the
    # last Sq rows of the full causal prefill.
    q, k, v = _qkv(18, 2, 30, 30, 4, 2, 8)
    full = oracle.attention(q, k, v, True, 0.4)
    for Sq in (1, 4, 29):
        part = oracle.attention(q[:, -Sq:], k, v, True, 0.4)
        np.testing.assert_allclose(part, full[:, -Sq:], rtol=0, atol=1e-12)


def test_kv_cache_example_fixture():
    g = json.load(open(os.path.join(GOLDEN, "kv_cache_token4.json")))
    n = g["n_cached_after_append"]
    q, k, _ = _qkv(19, 1, n, n, 1, 1, 8)
    p_full = oracle.attention_probs(q, k, 1.0, True, 0, 0)
    p_last = oracle.attention_probs(q[:, -1:], k, 1.0, True, 0, 0)
    assert list(p_last.shape) == g["score_shape"]
    np.testing.assert_allclose(p_last[0], p_full[-1], rtol=0, atol=1e-15)
    # rows 0..n-2 are unchanged when token n is appended
    p_prev = oracle.attention_probs(q[:, :-1], k[:, :-1], 1.0, True, 0, 0)
    np.testing.assert_allclose(p_full[:-1, :-1], p_prev, rtol=0, atol=1e-15)


def test_tp_demo_shape_fixture():
    g = json.load(open(os.path.join(GOLDEN, "tp_attention_demo_shape.json")))
    B, S, H = g["batch"], g["seq"], g["heads"]
    D = g["hidden"] // H
    r = _rng(20)
    q = r.standard_normal((B, S, H, D)).astype(np.float32)
    out = oracle.attention(q, q, q, False, 1.0 / math.sqrt(D), heads=[(0, 0)])
    assert list(out.reshape(B, S, H * D).shape) == g["expected_shape"]


def test_kv_append():
    r = _rng(21)
    kc, vc = r.standard_normal((2, 3, 6, 4)), r.standard_normal((2, 3, 6, 4))
    kn, vn = r.standard_normal((2, 3, 4)), r.standard_normal((2, 3, 4))
    k2, v2 = oracle.kv_append(kc, vc, kn, vn, np.array([5, 6]))
    np.testing.assert_array_equal(k2[0, :, 5], kn[0])
    np.testing.assert_array_equal(v2[0, :, 5], vn[0])
    np.testing.assert_array_equal(k2[1], kc[1])          # slot 6 is out of range
    np.testing.assert_array_equal(k2[0, :, :5], kc[0, :, :5])
