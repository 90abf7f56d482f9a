"""attn_prefill_ws (split-K over workgroups for small causal prefills) on the
GPU: the float64 oracle element by element, the workspace left ready for the
next call, repeatability, and the shapes that run as attn_prefill."""
import math

import numpy as np
import pytest

import oracle
import rope_causal_gqa_amd as R
from rope_causal_gqa_amd import workloads as W
from tests.gpu_helpers import announce, check, dev, host64

pytestmark = pytest.mark.gpu

CANARY = 0x5A


def _workspace(need, pad=4096):
    """Zeroed workspace of `need` bytes followed by `pad` canary bytes."""
    import torch
    ws = torch.zeros(need + pad, dtype=torch.uint8, device="cuda")
    ws[need:] = CANARY
    return ws


def _check_workspace(ws, need):
    """Counters (the first 4096 bytes of the workspace) back at zero, nothing
    written past the end."""
    import torch
    torch.cuda.synchronize()
    host = ws.cpu().numpy()
    assert np.all(host[need:] == CANARY), "write past the workspace"
    assert np.all(host[:min(need, 4096)] == 0), "counters not reset"


def test_full_size_all_heads():
    """One GPU's 8-query-head / 1-KV-head share of the 70B-shaped prefill
    (rope then attention), every head against the oracle."""
    import torch
    w = W.WORKLOADS["c4b"]
    announce(f"split prefill c4b full size, all {w.Hq} heads")
    q, k, v = W.prefill_inputs(w)
    qd, kd, vd = dev(q, w.dtype), dev(k, w.dtype), dev(v, w.dtype)
    R.rope_apply(qd, kd, None, w.theta, w.factor)
    need = R.attn_prefill_workspace_bytes(w.B, w.S, w.Hq, w.D, True)
    assert need > 0
    ws = _workspace(need)
    out = R.attn_prefill_ws(qd, kd, vd, causal=True, scale=w.scale, workspace=ws)
    _check_workspace(ws, need)
    got = host64(out)
    q64, k64 = oracle.rope_apply(W.to_f64(q, w.dtype), W.to_f64(k, w.dtype), None, w.theta, w.factor)
    ref = oracle.attention(q64, k64, W.to_f64(v, w.dtype), True, w.scale)
    for h in range(w.Hq):
        check(got[0, :, h], ref[0, :, h], w.dtype, f"split c4b h={h}")


SPLIT = [
    # B, S, Hq, Hkv, D (shapes the launcher would run on an unpaired grid, with at
    # least 16 units of work per workgroup): ragged last tile with several KV
    # heads, D=64, B > 1, Hkv = Hq, a ragged tail at B=3
    (1, 2100, 32, 4, 128),
    (1, 2048, 32, 4, 64),
    (4, 2048, 8, 1, 128),
    (2, 2048, 16, 16, 128),
    (3, 1700, 16, 8, 128),
]


@pytest.mark.parametrize("B,S,Hq,Hkv,D", SPLIT)
def test_split_shapes(B, S, Hq, Hkv, D):
    import torch
    announce(f"split prefill B={B} S={S} Hq={Hq} Hkv={Hkv} D={D}")
    seed = 31 + B * 7 + S * 13 + Hq * 17 + D
    q = W.random_case(seed, (B, S, Hq, D), "bf16")
    k = W.random_case(seed + 1, (B, S, Hkv, D), "bf16")
    v = W.random_case(seed + 2, (B, S, Hkv, D), "bf16")
    scale = 1.0 / math.sqrt(D)
    need = R.attn_prefill_workspace_bytes(B, S, Hq, D, True)
    assert need > 0
    ws = _workspace(need)
    n = B * S * Hq * D
    buf = torch.full((n + 2048,), 7.0, dtype=torch.bfloat16, device="cuda")
    out = buf[1024:1024 + n].view(B, S, Hq, D)
    qd, kd, vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    R.attn_prefill_ws(qd, kd, vd, out, causal=True, scale=scale, workspace=ws)
    _check_workspace(ws, need)
    assert torch.all(buf[:1024] == 7.0) and torch.all(buf[1024 + n:] == 7.0), "write outside out"
    first = out.clone()
    ref = oracle.attention(W.to_f64(q, "bf16"), W.to_f64(k, "bf16"), W.to_f64(v, "bf16"), True, scale)
    check(host64(out), ref, "bf16", f"split B={B} S={S} Hq={Hq} Hkv={Hkv} D={D}")
    # the same workspace again: the counters were left at zero, the result repeats bit for bit
    R.attn_prefill_ws(qd, kd, vd, out, causal=True, scale=scale, workspace=ws)
    _check_workspace(ws, need)
    assert torch.equal(out, first)


def test_repeatable_and_workspace_reuse_across_shapes():
    """Five calls give bitwise equal results (the merge runs in chunk order
    whichever chunk finishes last); a smaller problem then reuses the same
    workspace."""
    import torch
    w = W.WORKLOADS["c4b"]
    g = torch.Generator(device="cuda")
    g.manual_seed(12)
    q, k, v = (torch.randn((w.B, w.S, H, w.D), generator=g, device="cuda").to(torch.bfloat16)
               for H in (w.Hq, w.Hkv, w.Hkv))
    need = R.attn_prefill_workspace_bytes(w.B, w.S, w.Hq, w.D, True)
    ws = _workspace(need)
    ref = R.attn_prefill_ws(q, k, v, causal=True, scale=w.scale, workspace=ws)
    for _ in range(5):
        again = R.attn_prefill_ws(q, k, v, causal=True, scale=w.scale, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(again, ref)
    _check_workspace(ws, need)
    S2 = 4000
    q2, k2, v2 = (t[:, :S2].contiguous() for t in (q, k, v))
    small = R.attn_prefill_ws(q2, k2, v2, causal=True, scale=w.scale, workspace=ws)
    fresh = R.attn_prefill_ws(q2, k2, v2, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(small, fresh)
    ref2 = oracle.attention(host64(q2), host64(k2), host64(v2), True, w.scale, heads=[(0, 0), (0, 7)])
    got2 = host64(small)
    for h in (0, 7):
        check(got2[0, :, h], ref2[0, :, h], "bf16", f"split reuse S={S2} h={h}")


@pytest.mark.parametrize("B,S,Hq,Hkv,D,causal,dtype", [
    (1, 2048, 8, 2, 128, False, "bf16"),   # not causal
    (2, 1000, 32, 8, 128, True, "bf16"),   # fills the GPU with one workgroup per tile
    (1, 4096, 32, 8, 128, True, "bf16"),   # the paired 4-wave grid
    (1, 2100, 8, 1, 128, True, "bf16"),    # too little work per workgroup
    (1, 300, 4, 1, 64, True, "fp32"),
])
def test_runs_as_attn_prefill_otherwise(B, S, Hq, Hkv, D, causal, dtype):
    import torch
    announce(f"split prefill fallback B={B} S={S} Hq={Hq} causal={causal} {dtype}")
    assert dtype == "fp32" or R.attn_prefill_workspace_bytes(B, S, Hq, D, causal) == 0
    seed = 77 + S
    q = W.random_case(seed, (B, S, Hq, D), dtype)
    k = W.random_case(seed + 1, (B, S, Hkv, D), dtype)
    v = W.random_case(seed + 2, (B, S, Hkv, D), dtype)
    qd, kd, vd = dev(q, dtype), dev(k, dtype), dev(v, dtype)
    a = R.attn_prefill(qd, kd, vd, causal=causal, scale=D ** -0.5)
    b = R.attn_prefill_ws(qd, kd, vd, causal=causal, scale=D ** -0.5)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("S,Hq", [(16384, 4), (32768, 2)])
def test_long_sequence_sampled_rows(S, Hq):
    """Long sequences (64 and 128 query tiles per head, the most the plan
    takes): sampled rows against the oracle, each as a single query over its
    visible keys (the single-query form of the same attention)."""
    import torch
    B, Hkv, D = 1, 1, 128
    announce(f"split prefill long S={S} Hq={Hq}")
    assert R.attn_prefill_workspace_bytes(B, S, Hq, D, True) > 0
    seed = 700 + S
    q = W.random_case(seed, (B, S, Hq, D), "bf16")
    k = W.random_case(seed + 1, (B, S, Hkv, D), "bf16")
    v = W.random_case(seed + 2, (B, S, Hkv, D), "bf16")
    out = R.attn_prefill_ws(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), causal=True, scale=D ** -0.5)
    torch.cuda.synchronize()
    got = host64(out)
    assert np.all(np.isfinite(got))
    k64 = np.transpose(W.to_f64(k, "bf16"), (0, 2, 1, 3))     # [B, Hkv, S, D] cache layout
    v64 = np.transpose(W.to_f64(v, "bf16"), (0, 2, 1, 3))
    q64 = W.to_f64(q, "bf16")
    for i in [0, 255, 256, 4095, S // 2 + 13, S - 257, S - 1]:
        ref = oracle.attention_cache(q64[:, i:i + 1], k64, v64, np.full(B, i + 1), True, D ** -0.5)
        check(got[:, i:i + 1], ref, "bf16", f"split long S={S} row {i}")
