"""attn_prefill_cache_ws (stream-K for causal chunks against a KV cache) on
the GPU: the float64 oracle on every head, sequences shorter than the cache
(the plan counts every sequence as full), repeatability, the workspace left
ready for the next call, and the shapes that run as attn_prefill_cache."""
import math

import numpy as np
import pytest

import oracle
import rope_causal_gqa_amd as R
from rope_causal_gqa_amd import workloads as W
from tests.gpu_helpers import announce, check, dev, host64

pytestmark = pytest.mark.gpu

CANARY = 0x5A


def _case(seed, B, Sq, Hq, Hkv, D, max_kv):
    q = W.random_case(seed, (B, Sq, Hq, D), "bf16")
    kc = W.random_case(seed + 1, (B, Hkv, max_kv, D), "bf16")
    vc = W.random_case(seed + 2, (B, Hkv, max_kv, D), "bf16")
    return q, kc, vc


CASES = [
    # B, Sq, Hq, Hkv, D, max_kv, kv_lens (shapes whose key-group grid would not
    # fill the GPU, with at least 16 units of work per workgroup)
    (1, 512, 32, 32, 128, 8192, [8192]),          # a chunk of 512 after 7680 cached tokens
    (2, 512, 16, 16, 128, 4608, [3000, 4608]),    # one sequence shorter than the cache
    (2, 512, 16, 8, 64, 4608, [512, 100]),        # D=64; a chunk alone; a sequence shorter than the chunk
    (2, 512, 16, 16, 128, 4608, [0, -5]),         # empty sequences: zero rows
    (1, 1024, 16, 4, 128, 6144, [6144]),          # GQA, four query tiles
    (2, 700, 16, 16, 128, 3000, [3000, 2999]),    # ragged last query tile
]


@pytest.mark.parametrize("B,Sq,Hq,Hkv,D,max_kv,lens", CASES)
def test_cache_split_against_oracle(B, Sq, Hq, Hkv, D, max_kv, lens):
    import torch
    announce(f"cache split B={B} Sq={Sq} Hq={Hq} Hkv={Hkv} D={D} max_kv={max_kv} lens={lens}")
    need = R.attn_prefill_cache_workspace_bytes(B, Sq, Hq, D, max_kv, True, 0)
    assert need > 0
    q, kc, vc = _case(61 + Sq + max_kv + Hkv + D, B, Sq, Hq, Hkv, D, max_kv)
    ws = torch.zeros(need + 4096, dtype=torch.uint8, device="cuda")
    ws[need:] = CANARY
    n = q.size
    buf = torch.full((n + 2048,), 7.0, dtype=torch.bfloat16, device="cuda")
    out = buf[1024:1024 + n].view(q.shape)
    lens_d = torch.tensor(lens, dtype=torch.int32, device="cuda")
    qd, kd, vd = dev(q, "bf16"), dev(kc, "bf16"), dev(vc, "bf16")
    R.attn_prefill_cache_ws(qd, kd, vd, lens_d, out, causal=True, scale=1.0 / math.sqrt(D), workspace=ws)
    torch.cuda.synchronize()
    assert torch.all(buf[:1024] == 7.0) and torch.all(buf[1024 + n:] == 7.0), "write outside out"
    host = ws.cpu().numpy()
    assert np.all(host[need:] == CANARY), "write past the workspace"
    assert np.all(host[:4096] == 0), "counters not reset"
    first = out.clone()
    ref = oracle.attention_cache(W.to_f64(q, "bf16"), W.to_f64(kc, "bf16"), W.to_f64(vc, "bf16"),
                                 np.array(lens), True, 1.0 / math.sqrt(D))
    got = host64(out)
    for b in range(B):
        for h in range(Hq):
            check(got[b, :, h], ref[b, :, h], "bf16", f"cache split lens={lens} b={b} h={h}")
    # again with the same workspace: bit for bit
    R.attn_prefill_cache_ws(qd, kd, vd, lens_d, out, causal=True, scale=1.0 / math.sqrt(D), workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, first)


def test_full_cache_equals_plain_stream_k():
    """A chunk that is the whole sequence (Sq = kv_len = max_kv) is a plain
    prefill: the same plan, and the same bits as attn_prefill_ws."""
    import torch
    announce("cache split: Sq = max_kv against attn_prefill_ws")
    B, S, Hq, Hkv, D = 1, 8192, 2, 1, 128
    q = W.random_case(5, (B, S, Hq, D), "bf16")
    k = W.random_case(6, (B, S, Hkv, D), "bf16")
    v = W.random_case(7, (B, S, Hkv, D), "bf16")
    qd, kd, vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    kc, vc = kd.permute(0, 2, 1, 3).contiguous(), vd.permute(0, 2, 1, 3).contiguous()
    lens = torch.full((B,), S, dtype=torch.int32, device="cuda")
    assert R.attn_prefill_cache_workspace_bytes(B, S, Hq, D, S, True, 0) == R.attn_prefill_workspace_bytes(B, S, Hq, D)
    a = R.attn_prefill_cache_ws(qd, kc, vc, lens, causal=True, scale=D ** -0.5)
    b = R.attn_prefill_ws(qd, kd, vd, causal=True, scale=D ** -0.5)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("causal,window,dtype,Hq", [(1, 1024, "bf16", 16), (0, 0, "bf16", 16), (1, 0, "fp32", 16),
                                                  (1, 0, "bf16", 32)])   # the last: a full key-group grid
def test_runs_as_attn_prefill_cache_otherwise(causal, window, dtype, Hq):
    import torch
    announce(f"cache split fallback causal={causal} window={window} {dtype} Hq={Hq}")
    B, Sq, Hkv, D, max_kv = 2, 512, Hq, 128, 4608
    if dtype == "fp32":
        B, Sq, Hq, Hkv, D, max_kv = 1, 300, 4, 1, 64, 700
    assert dtype == "fp32" or R.attn_prefill_cache_workspace_bytes(B, Sq, Hq, D, max_kv, causal, window) == 0
    q = W.random_case(90, (B, Sq, Hq, D), dtype)
    kc = W.random_case(91, (B, Hkv, max_kv, D), dtype)
    vc = W.random_case(92, (B, Hkv, max_kv, D), dtype)
    qd, kd, vd = dev(q, dtype), dev(kc, dtype), dev(vc, dtype)
    lens = torch.tensor([max_kv, max_kv - 7][:B], dtype=torch.int32, device="cuda")
    a = R.attn_prefill_cache(qd, kd, vd, lens, causal=causal, scale=D ** -0.5, window=window)
    b = R.attn_prefill_cache_ws(qd, kd, vd, lens, causal=causal, scale=D ** -0.5, window=window)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
