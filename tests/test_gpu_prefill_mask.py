"""attn_prefill_masked on the GPU against the float64 oracle's additive mask:
key padding with and without the causal mask, per-head finite biases,
fully masked rows, row strides beyond S (aligned and not), fp32, every
prefill grid (8-wave, 4-wave, two and four key groups); and bit for bit: a zero
mask gives attn_prefill's result, a -inf upper triangle without the causal
flag gives the causal result."""
import math

import numpy as np
import pytest

import oracle
import rope_causal_gqa_amd as R
from rope_causal_gqa_amd import workloads as W
from tests.gpu_helpers import announce, check, dev, host64

pytestmark = pytest.mark.gpu


def _bf16_bits(x):
    """float64 -> bf16 bit patterns (round to nearest even), keeping infinities."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r = np.where(np.isinf(f), (f.view(np.uint32) >> 16).astype(np.uint16), r)
    return r


def _mask_dev(m, dtype):
    return dev(_bf16_bits(m) if dtype == "bf16" else m.astype(np.float32), dtype)


def _mask_host(m, dtype):
    """the values the GPU sees, as float64"""
    if dtype == "bf16":
        return (_bf16_bits(m).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return m.astype(np.float32).astype(np.float64)


def _padding(B, S, L, lens, left=False):
    m = np.zeros((B, 1, S, L))
    for b, n in enumerate(lens):
        if left:
            m[b, :, :, :S - n] = -np.inf
        else:
            m[b, :, :, n:S] = -np.inf
    return m


def _alibi(B, Hq, S, L):
    slopes = np.array([2.0 ** (-8.0 * (h + 1) / Hq) for h in range(Hq)])
    i, j = np.arange(S)[:, None], np.arange(L)[None, :]
    return np.broadcast_to(-slopes[None, :, None, None] * np.abs(i - j)[None, None], (B, Hq, S, L)).copy()


CASES = [
    # B, S, Hq, Hkv, D, causal, dtype, mask kind, row stride
    (2, 300, 8, 2, 128, True, "bf16", "pad", 300),
    (2, 300, 8, 2, 128, False, "bf16", "pad_left", 304),
    (1, 77, 4, 4, 64, False, "bf16", "alibi", 77),
    (2, 129, 8, 1, 128, True, "bf16", "alibi", 131),       # row stride not a multiple of 4
    (2, 70, 4, 2, 64, True, "fp32", "pad", 70),
    (1, 97, 4, 2, 128, False, "fp32", "alibi", 99),
    (2, 200, 4, 2, 128, False, "bf16", "dead_rows", 200),
    (2, 2048, 32, 8, 128, True, "bf16", "pad", 2048),      # 8-wave grid, mask tiles staged in LDS
    (2, 2048, 32, 8, 128, True, "bf16", "alibi", 2056),    # same, per-head mask, padded rows
    (2, 2048, 32, 8, 64, True, "bf16", "pad_left", 2052),  # rows not a multiple of 8: another grid
    (1, 2100, 8, 1, 128, True, "bf16", "pad", 2100),       # four key groups
    (1, 2100, 16, 2, 64, True, "bf16", "alibi", 2104),     # two key groups
]


@pytest.mark.parametrize("B,S,Hq,Hkv,D,causal,dtype,kind,ld", CASES)
def test_masked_prefill(B, S, Hq, Hkv, D, causal, dtype, kind, ld):
    import torch
    announce(f"masked prefill B={B} S={S} Hq={Hq} Hkv={Hkv} D={D} causal={causal} {dtype} {kind} ld={ld}")
    seed = 17 + S + Hq + D
    q = W.random_case(seed, (B, S, Hq, D), dtype)
    k = W.random_case(seed + 1, (B, S, Hkv, D), dtype)
    v = W.random_case(seed + 2, (B, S, Hkv, D), dtype)
    if kind == "pad":
        m = _padding(B, S, ld, [S - 37 * b - 5 for b in range(B)])
    elif kind == "pad_left":
        m = _padding(B, S, ld, [S - 29 * b - 11 for b in range(B)], left=True)
    elif kind == "alibi":
        m = _alibi(B, Hq, S, ld)
    else:  # a few rows with no visible key, the rest a random bias
        m = np.random.Generator(np.random.PCG64(seed)).standard_normal((B, 1, S, ld))
        m[:, :, ::17, :] = -np.inf
    m[..., S:] = np.nan                                      # padding past S must never be read
    scale = 1.0 / math.sqrt(D)
    out = R.attn_prefill_masked(dev(q, dtype), dev(k, dtype), dev(v, dtype), _mask_dev(m, dtype), causal=causal,
                                scale=scale)
    torch.cuda.synchronize()
    got = host64(out)
    assert np.all(np.isfinite(got))
    mh = _mask_host(m[..., :S], dtype)
    q64, k64, v64 = W.to_f64(q, dtype), W.to_f64(k, dtype), W.to_f64(v, dtype)
    if B * S * Hq <= 64 * 1024:
        check(got, oracle.attention(q64, k64, v64, causal, scale, mask=mh), dtype, f"masked {kind}")
    else:
        heads = [(0, 0), (B - 1, Hq - 1), (0, Hq // 2)]
        ref = oracle.attention(q64, k64, v64, causal, scale, heads=heads, mask=mh)
        for b, h in heads:
            check(got[b, :, h], ref[b, :, h], dtype, f"masked {kind} b={b} h={h}")
    if kind == "dead_rows":
        assert np.all(got[:, ::17] == 0.0)


@pytest.mark.parametrize("B,S,Hq,Hkv,same_split", [(2, 2048, 32, 32, True), (1, 1024, 64, 8, True),
                                                   (1, 2100, 8, 1, False), (1, 300, 8, 2, False)])
def test_masked_prefill_bitwise_pins(B, S, Hq, Hkv, same_split):
    """A zero mask reproduces attn_prefill bit for bit on each grid (8-wave,
    4-wave, four and two key groups).  A -inf upper triangle without the
    causal flag reproduces the causal result bit for bit where the keys are
    not split across groups; with key groups the non-causal call splits the
    whole key range (and may pick the other grid), so the sums are grouped
    differently and agree to rounding."""
    import torch
    announce(f"masked prefill bitwise pins B={B} S={S} Hq={Hq} Hkv={Hkv}")
    D = 128
    q, k, v = (dev(W.random_case(s, (B, S, h, D), "bf16"), "bf16") for s, h in ((61, Hq), (62, Hkv), (63, Hkv)))
    zero = torch.zeros((B, 1, S, S), dtype=torch.bfloat16, device="cuda")
    tri = torch.triu(torch.full((S, S), float("-inf"), device="cuda"), diagonal=1).to(torch.bfloat16)
    tri = tri.expand(B, 1, S, S).contiguous()
    ref = R.attn_prefill(q, k, v, causal=True, scale=D ** -0.5)
    got0 = R.attn_prefill_masked(q, k, v, zero, causal=True, scale=D ** -0.5)
    got1 = R.attn_prefill_masked(q, k, v, tri, causal=False, scale=D ** -0.5)
    torch.cuda.synchronize()
    assert torch.equal(got0, ref), "zero mask changes the causal result"
    if same_split:
        assert torch.equal(got1, ref), "a -inf upper triangle differs from the causal mask"
    else:
        d = (got1.float() - ref.float()).abs().max().item()
        assert d <= 8e-3, f"a -inf upper triangle differs from the causal mask by {d}"
