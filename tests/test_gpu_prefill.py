"""attn_prefill (and the rope -> prefill path) on the GPU against the float64 oracle."""
import math

import numpy as np
import pytest

import oracle
import rope_causal_gqa_amd as R
from rope_causal_gqa_amd import workloads as W
from tests.gpu_helpers import announce, check, dev, host64

pytestmark = pytest.mark.gpu


def _path(w, q, k, v, heads=None):
    """Run rope (if the workload has it) + prefill on the GPU and in the oracle."""
    import torch
    qd, kd, vd = dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype)
    if w.rope:
        R.rope_apply(qd, kd, None, w.theta, w.factor)
    out = R.attn_prefill(qd, kd, vd, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    got = host64(out)
    q64, k64, v64 = W.to_f64(q, w.dtype), W.to_f64(k, w.dtype), W.to_f64(v, w.dtype)
    if heads is not None:
        # rotate only what the sampled heads read
        G = w.Hq // w.Hkv
        qs = sorted({h for _, h in heads})
        ks = sorted({h // G for _, h in heads})
        q64 = q64.copy()
        k64 = k64.copy()
        if w.rope:
            qr, kr = oracle.rope_apply(q64[:, :, qs], k64[:, :, ks], None, w.theta, w.factor)
            q64[:, :, qs] = qr
            k64[:, :, ks] = kr
    elif w.rope:
        q64, k64 = oracle.rope_apply(q64, k64, None, w.theta, w.factor)
    ref = oracle.attention(q64, k64, v64, w.causal, w.scale, heads=heads)
    return got, ref


@pytest.mark.parametrize("name", ["c1", "c2a", "c2b"])
def test_prefill_small_workloads(name):
    w = W.WORKLOADS[name]
    announce(f"prefill {name}")
    got, ref = _path(w, *W.prefill_inputs(w))
    check(got, ref, w.dtype, f"rope+prefill {name}")


@pytest.mark.parametrize("name", ["c3", "c4a", "c4b"])
def test_prefill_full_size_all_heads(name):
    """The LLaMA-sized prefills, every (batch, head) slice element by element."""
    w = W.WORKLOADS[name]
    announce(f"prefill {name} full size, all {w.B * w.Hq} heads")
    got, ref = _path(w, *W.prefill_inputs(w))
    for b in range(w.B):
        for h in range(w.Hq):
            check(got[b, :, h], ref[b, :, h], w.dtype, f"{name} b={b} h={h}")


EDGE = [
    # B, S, Hq, Hkv, D, causal, dtype
    (1, 1, 1, 1, 128, True, "bf16"),
    (3, 63, 4, 1, 128, True, "bf16"),
    (1, 64, 2, 2, 128, True, "bf16"),
    (2, 65, 8, 2, 128, True, "bf16"),
    (1, 127, 4, 4, 128, False, "bf16"),
    (1, 129, 16, 1, 128, True, "bf16"),
    (1, 200, 6, 3, 64, True, "bf16"),
    (2, 300, 4, 2, 64, False, "bf16"),
    (1, 517, 2, 1, 128, True, "bf16"),
    (1, 1, 2, 1, 64, True, "fp32"),
    (3, 63, 4, 2, 64, True, "fp32"),
    (1, 97, 4, 1, 128, False, "fp32"),
    (2, 130, 2, 2, 128, True, "fp32"),
]


@pytest.mark.parametrize("B,S,Hq,Hkv,D,causal,dtype", EDGE)
def test_prefill_edges(B, S, Hq, Hkv, D, causal, dtype):
    import torch
    announce(f"prefill edge B={B} S={S} Hq={Hq} Hkv={Hkv} D={D} causal={causal} {dtype}")
    seed = B * 7 + S * 13 + Hq * 17 + D
    q = W.random_case(seed, (B, S, Hq, D), dtype)
    k = W.random_case(seed + 1, (B, S, Hkv, D), dtype)
    v = W.random_case(seed + 2, (B, S, Hkv, D), dtype)
    scale = 1.0 / math.sqrt(D)
    qd, kd, vd = dev(q, dtype), dev(k, dtype), dev(v, dtype)
    # guard canaries around the output
    n = B * S * Hq * D
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    buf = torch.full((n + 2048,), 7.0, dtype=tdt, device="cuda")
    out = buf[1024:1024 + n].view(B, S, Hq, D)
    R.attn_prefill(qd, kd, vd, out, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert torch.all(buf[:1024] == 7.0) and torch.all(buf[1024 + n:] == 7.0), "write outside out"
    ref = oracle.attention(W.to_f64(q, dtype), W.to_f64(k, dtype), W.to_f64(v, dtype), causal, scale)
    check(host64(out), ref, dtype, f"edge B={B} S={S} Hq={Hq} Hkv={Hkv} D={D} c={causal}")


# Causal grids with at least 512 paired 256-row tiles take the 8-wave kernel:
# ragged S, an odd number of 256-row tiles (one unpaired middle tile), D=64.
BIG = [
    # B, S, Hq, Hkv, D, heads sampled
    (8, 1000, 32, 8, 128, [(0, 0), (3, 13), (7, 31)]),
    (4, 1100, 64, 8, 128, [(0, 1), (2, 40), (3, 63)]),
    (4, 777, 64, 8, 64, [(0, 0), (1, 22), (3, 57)]),
]


@pytest.mark.parametrize("B,S,Hq,Hkv,D,heads", BIG)
def test_prefill_eight_wave_grid(B, S, Hq, Hkv, D, heads):
    import torch
    announce(f"prefill 8-wave grid B={B} S={S} Hq={Hq} Hkv={Hkv} D={D}")
    seed = 5 + B * 7 + S * 13 + Hq * 17 + D
    q = W.random_case(seed, (B, S, Hq, D), "bf16")
    k = W.random_case(seed + 1, (B, S, Hkv, D), "bf16")
    v = W.random_case(seed + 2, (B, S, Hkv, D), "bf16")
    scale = 1.0 / math.sqrt(D)
    n = B * S * Hq * D
    buf = torch.full((n + 2048,), 7.0, dtype=torch.bfloat16, device="cuda")
    out = buf[1024:1024 + n].view(B, S, Hq, D)
    R.attn_prefill(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), out, causal=True, scale=scale)
    torch.cuda.synchronize()
    assert torch.all(buf[:1024] == 7.0) and torch.all(buf[1024 + n:] == 7.0), "write outside out"
    got = host64(out)
    assert np.all(np.isfinite(got))
    ref = oracle.attention(W.to_f64(q, "bf16"), W.to_f64(k, "bf16"), W.to_f64(v, "bf16"), True, scale,
                           heads=heads)
    for b, h in heads:
        check(got[b, :, h], ref[b, :, h], "bf16", f"8-wave B={B} S={S} b={b} h={h}")


# Grids too small for 512 workgroups of 4 waves run one 8-wave workgroup per
# CU, in two key groups over 128-row tiles or four over 64-row tiles,
# whichever the launcher estimates to finish first.  These shapes take the
# four-group kernel (paired causal tiles, unpaired causal tiles with D=64,
# non-causal; ragged tails) and, last, the two-group one.
FOUR = [
    # B, S, Hq, Hkv, D, causal
    (1, 4000, 8, 2, 128, True),
    (1, 2100, 8, 1, 64, True),
    (1, 2000, 8, 2, 128, False),
    (1, 2100, 16, 2, 128, True),
]


@pytest.mark.parametrize("B,S,Hq,Hkv,D,causal", FOUR)
def test_prefill_key_groups(B, S, Hq, Hkv, D, causal):
    import torch
    announce(f"prefill key groups B={B} S={S} Hq={Hq} Hkv={Hkv} D={D} causal={causal}")
    seed = 9 + B * 7 + S * 13 + Hq * 17 + D
    q = W.random_case(seed, (B, S, Hq, D), "bf16")
    k = W.random_case(seed + 1, (B, S, Hkv, D), "bf16")
    v = W.random_case(seed + 2, (B, S, Hkv, D), "bf16")
    scale = 1.0 / math.sqrt(D)
    n = B * S * Hq * D
    buf = torch.full((n + 2048,), 7.0, dtype=torch.bfloat16, device="cuda")
    out = buf[1024:1024 + n].view(B, S, Hq, D)
    R.attn_prefill(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), out, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert torch.all(buf[:1024] == 7.0) and torch.all(buf[1024 + n:] == 7.0), "write outside out"
    ref = oracle.attention(W.to_f64(q, "bf16"), W.to_f64(k, "bf16"), W.to_f64(v, "bf16"), causal, scale)
    check(host64(out), ref, "bf16", f"key groups B={B} S={S} Hq={Hq} D={D} c={causal}")


@pytest.mark.parametrize("name", ["c2b", "c3", "c4b"])
def test_prefill_deterministic(name):
    """Repeated launches give bitwise equal results (c3 takes the 8-wave
    kernel, c2b the 4-wave one, c4b the one with four key groups)."""
    import torch
    w = W.WORKLOADS[name]
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    q, k, v = (torch.randn((w.B, w.S, H, w.D), generator=g, device="cuda").to(torch.bfloat16)
               for H in (w.Hq, w.Hkv, w.Hkv))
    ref = R.attn_prefill(q, k, v, causal=True, scale=w.scale)
    for _ in range(5):
        again = R.attn_prefill(q, k, v, causal=True, scale=w.scale)
        torch.cuda.synchronize()
        assert torch.equal(again, ref)


def test_prefill_on_side_stream():
    import torch
    w = W.WORKLOADS["c2a"]
    q, k, v = (dev(a, "bf16") for a in W.prefill_inputs(w))
    ref = R.attn_prefill(q, k, v, causal=False, scale=w.scale)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out = R.attn_prefill(q, k, v, causal=False, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


@pytest.mark.parametrize("dtype,S,D", [("bf16", 1000, 128), ("bf16", 700, 64), ("fp32", 300, 64)])
def test_prefill_growing_scores(dtype, S, D):
    """Scores that grow along the sequence move the running max by far more
    than the lazy-rescale margin on almost every key tile, so the rescale of
    the accumulators (rare on N(0,1) inputs) runs throughout."""
    import torch
    announce(f"prefill growing scores {dtype} S={S} D={D}")
    r = np.random.Generator(np.random.PCG64(S + D))
    u = r.standard_normal(D)
    u /= np.linalg.norm(u)
    B, Hq, Hkv = 1, 4, 2
    # bf16: score growth per 64-key tile ~ 30 * 64/12 * scale = 14-20 (natural log
    # units), well past the lazy-rescale margin of 2^8.  fp32 (no lazy rescale; it
    # moves its max on every larger score) uses amplitude 10 so scores stay within
    # ~40, where fp32 score rounding (proportional to |score|) keeps the 1e-5 bar.
    amp = 30.0 if dtype == "bf16" else 10.0
    q = (amp * u + 0.3 * r.standard_normal((B, S, Hq, D)))
    ramp = (np.arange(S) / 12.0)[None, :, None, None]
    k = ramp * u + 0.3 * r.standard_normal((B, S, Hkv, D))
    v = r.standard_normal((B, S, Hkv, D))
    if dtype == "bf16":
        q, k, v = (W.round_bf16(a) for a in (q, k, v))
    else:
        q, k, v = (a.astype(np.float32) for a in (q, k, v))
    scale = 1.0 / math.sqrt(D)
    out = R.attn_prefill(dev(q, dtype), dev(k, dtype), dev(v, dtype), causal=True, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.attention(W.to_f64(q, dtype), W.to_f64(k, dtype), W.to_f64(v, dtype), True, scale)
    check(host64(out), ref, dtype, f"growing scores {dtype} S={S} D={D}")


@pytest.mark.parametrize("B,S,Hq,Hkv,D,causal", [(1, 16384, 4, 1, 128, True), (1, 12000, 8, 2, 64, False)])
def test_prefill_long_sequence_sampled_rows(B, S, Hq, Hkv, D, causal):
    """A long sequence (many query tiles, 32-bit tile offsets far into K/V):
    sampled rows against the oracle, each as a single query over its visible
    keys (the single-query form of the same attention, `attention_cache`)."""
    import torch
    announce(f"prefill long B={B} S={S} Hq={Hq} Hkv={Hkv} D={D} causal={causal}")
    seed = 900 + S
    q = W.random_case(seed, (B, S, Hq, D), "bf16")
    k = W.random_case(seed + 1, (B, S, Hkv, D), "bf16")
    v = W.random_case(seed + 2, (B, S, Hkv, D), "bf16")
    out = R.attn_prefill(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), causal=causal, scale=D ** -0.5)
    torch.cuda.synchronize()
    got = host64(out)
    assert np.all(np.isfinite(got))
    k64 = np.transpose(W.to_f64(k, "bf16"), (0, 2, 1, 3))     # [B, Hkv, S, D] cache layout
    v64 = np.transpose(W.to_f64(v, "bf16"), (0, 2, 1, 3))
    q64 = W.to_f64(q, "bf16")
    rows = [0, 1, 63, 64, 4095, 8191, S // 2 + 17, S - 65, S - 2, S - 1]
    for i in rows:
        L = i + 1 if causal else S
        ref = oracle.attention_cache(q64[:, i:i + 1], k64, v64, np.full(B, L), causal, D ** -0.5)
        # with causal, the single query at position L-1 is row i; without, it sees all S keys
        check(got[:, i:i + 1], ref, "bf16", f"long row {i}")
