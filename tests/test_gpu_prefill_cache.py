"""attn_prefill_cache (chunked / variable-length prefill against a KV cache,
optional causal sliding window) on the GPU against the float64 oracle."""
import math

import numpy as np
import pytest

import oracle
import rope_causal_gqa_amd as R
from rope_causal_gqa_amd import workloads as W
from tests.gpu_helpers import announce, check, dev, host64

pytestmark = pytest.mark.gpu


def _case(seed, B, Sq, Hq, Hkv, D, max_kv, dtype):
    q = W.random_case(seed, (B, Sq, Hq, D), dtype)
    kc = W.random_case(seed + 1, (B, Hkv, max_kv, D), dtype)
    vc = W.random_case(seed + 2, (B, Hkv, max_kv, D), dtype)
    return q, kc, vc


def _run(q, kc, vc, lens, causal, window, dtype, D):
    import torch
    B, Sq, Hq, _ = q.shape
    n = q.size
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    buf = torch.full((n + 2048,), 7.0, dtype=tdt, device="cuda")   # canaries around out
    out = buf[1024:1024 + n].view(q.shape)
    lens_d = torch.tensor(lens, dtype=torch.int32, device="cuda")
    R.attn_prefill_cache(dev(q, dtype), dev(kc, dtype), dev(vc, dtype), lens_d, out, causal=causal,
                         scale=1.0 / math.sqrt(D), window=window)
    torch.cuda.synchronize()
    assert torch.all(buf[:1024] == 7.0) and torch.all(buf[1024 + n:] == 7.0), "write outside out"
    return host64(out)


CASES = [
    # B, Sq, Hq, Hkv, D, max_kv, kv_lens, causal, window, dtype
    (2, 100, 8, 2, 128, 800, [700, 333], 1, 0, "bf16"),        # chunk after a long context, ragged tiles
    (3, 64, 4, 1, 128, 256, [30, 64, 200], 1, 0, "bf16"),      # first rows of seq 0 see no key
    (3, 40, 4, 2, 64, 96, [0, 96, 500], 1, 0, "bf16"),         # empty cache; length past max_kv clamped
    (2, 40, 4, 2, 64, 96, [-7, 50], 1, 0, "bf16"),             # negative length: an empty cache
    (2, 77, 8, 8, 128, 160, [150, 1], 0, 0, "bf16"),           # non-causal
    (2, 300, 8, 2, 128, 1100, [300, 1000], 1, 64, "bf16"),     # sliding window
    (1, 129, 4, 1, 64, 129, [129], 1, 1, "bf16"),              # window 1: own value
    (2, 200, 4, 2, 128, 400, [260, 400], 1, 5000, "bf16"),     # window longer than the cache
    (2, 200, 4, 2, 128, 400, [10, 400], 1, 2147483647, "bf16"),  # int32-max window, fewer keys than queries
    (2, 1, 16, 2, 128, 700, [513, 700], 1, 0, "bf16"),         # one token: a decode step
    (1, 513, 2, 1, 128, 1500, [1500], 1, 300, "bf16"),         # window with tile-unaligned edges
    (1, 2100, 8, 1, 128, 3000, [2900], 1, 0, "bf16"),          # four key groups over 64-row tiles
    (1, 3000, 4, 2, 64, 3100, [3100], 1, 1500, "bf16"),        # four key groups, window
    (2, 2000, 4, 2, 128, 1900, [1900, 1000], 0, 0, "bf16"),    # four key groups, non-causal
    (1, 2100, 16, 2, 64, 2600, [2500], 1, 700, "bf16"),        # two key groups, window
    (2, 70, 4, 2, 64, 200, [150, 70], 1, 0, "fp32"),
    (2, 33, 8, 2, 128, 120, [20, 120], 1, 17, "fp32"),
    (1, 50, 2, 1, 64, 90, [90], 0, 0, "fp32"),
]


@pytest.mark.parametrize("B,Sq,Hq,Hkv,D,max_kv,lens,causal,window,dtype", CASES)
def test_prefill_cache_parity(B, Sq, Hq, Hkv, D, max_kv, lens, causal, window, dtype):
    announce(f"prefill_cache B={B} Sq={Sq} Hq={Hq} Hkv={Hkv} D={D} lens={lens} causal={causal} window={window} {dtype}")
    seed = 3 + B * 7 + Sq * 13 + Hq * 17 + D + window
    q, kc, vc = _case(seed, B, Sq, Hq, Hkv, D, max_kv, dtype)
    got = _run(q, kc, vc, lens, causal, window, dtype, D)
    ref = oracle.attention_cache(W.to_f64(q, dtype), W.to_f64(kc, dtype), W.to_f64(vc, dtype), np.array(lens),
                                 bool(causal), 1.0 / math.sqrt(D), window=window)
    check(got, ref, dtype, f"prefill_cache lens={lens} w={window}")


@pytest.mark.parametrize("B,Sq,Hq,Hkv,D,lens,window", [
    (2, 2048, 64, 8, 128, [4096, 3000], 0),      # 8-wave kernel, chunk against a long context
    (2, 2048, 64, 8, 128, [2048, 4000], 1024),   # 4-wave kernel, short sliding window
    (2, 2048, 64, 8, 128, [2048, 4000], 2500),   # 8-wave kernel, sliding window
])
def test_prefill_cache_large_all_heads(B, Sq, Hq, Hkv, D, lens, window):
    announce(f"prefill_cache large B={B} Sq={Sq} Hq={Hq} lens={lens} window={window}")
    max_kv = max(lens)
    q, kc, vc = _case(91 + window, B, Sq, Hq, Hkv, D, max_kv, "bf16")
    got = _run(q, kc, vc, lens, 1, window, "bf16", D)
    ref = oracle.attention_cache(W.to_f64(q, "bf16"), W.to_f64(kc, "bf16"), W.to_f64(vc, "bf16"), np.array(lens),
                                 True, 1.0 / math.sqrt(D), window=window)
    for b in range(B):
        for h in range(Hq):
            check(got[b, :, h], ref[b, :, h], "bf16", f"large b={b} h={h}")


@pytest.mark.parametrize("B,S,Hq,Hkv,D,dtype", [(2, 130, 8, 2, 128, "bf16"), (2, 1000, 64, 8, 128, "bf16"),
                                                 (1, 70, 4, 2, 64, "fp32")])
def test_full_chunk_equals_attn_prefill(B, S, Hq, Hkv, D, dtype):
    """Sq == kv_len with the cache holding the same K/V: the same kernel walks
    the same tiles, so the result equals attn_prefill bit for bit."""
    import torch
    announce(f"prefill_cache == attn_prefill B={B} S={S} Hq={Hq} {dtype}")
    seed = 500 + S
    q = dev(W.random_case(seed, (B, S, Hq, D), dtype), dtype)
    k = dev(W.random_case(seed + 1, (B, S, Hkv, D), dtype), dtype)
    v = dev(W.random_case(seed + 2, (B, S, Hkv, D), dtype), dtype)
    ref = R.attn_prefill(q, k, v, causal=True, scale=D ** -0.5)
    kc = k.permute(0, 2, 1, 3).contiguous()
    vc = v.permute(0, 2, 1, 3).contiguous()
    lens = torch.full((B,), S, dtype=torch.int32, device="cuda")
    got = R.attn_prefill_cache(q, kc, vc, lens, causal=True, scale=D ** -0.5)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)


def test_single_token_matches_decode():
    import torch
    announce("prefill_cache Sq=1 vs attn_decode")
    B, Hq, Hkv, D, max_kv = 4, 32, 4, 128, 900
    q, kc, vc = _case(77, B, 1, Hq, Hkv, D, max_kv, "bf16")
    lens = torch.tensor([1, 64, 511, 900], dtype=torch.int32, device="cuda")
    qd, kd, vd = dev(q, "bf16"), dev(kc, "bf16"), dev(vc, "bf16")
    a = R.attn_prefill_cache(qd, kd, vd, lens, causal=True, scale=D ** -0.5)
    d = R.attn_decode(qd.view(B, Hq, D), kd, vd, lens, scale=D ** -0.5)
    torch.cuda.synchronize()
    check(host64(a)[:, 0], host64(d), "bf16", "prefill_cache(Sq=1) vs decode")


def test_prefill_cache_deterministic():
    import torch
    B, Sq, Hq, Hkv, D, max_kv = 2, 512, 32, 8, 128, 3000
    q, kc, vc = _case(5, B, Sq, Hq, Hkv, D, max_kv, "bf16")
    qd, kd, vd = dev(q, "bf16"), dev(kc, "bf16"), dev(vc, "bf16")
    lens = torch.tensor([3000, 1700], dtype=torch.int32, device="cuda")
    ref = R.attn_prefill_cache(qd, kd, vd, lens, scale=D ** -0.5, window=700)
    for _ in range(3):
        again = R.attn_prefill_cache(qd, kd, vd, lens, scale=D ** -0.5, window=700)
        torch.cuda.synchronize()
        assert torch.equal(again, ref)
