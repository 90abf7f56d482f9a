"""rope_attn_prefill / rope_attn_decode (rotation fused with attention) on the
GPU: against the float64 oracle, and bit for bit against the separate calls
(rope_apply + attn_prefill; rope_apply + kv_append + attn_decode), which use
the same cos/sin values and the same arithmetic and rounding."""
import numpy as np
import pytest

import oracle
import rope_causal_gqa_amd as R
from rope_causal_gqa_amd import workloads as W
from tests.gpu_helpers import announce, check, dev, host64

pytestmark = pytest.mark.gpu


def _i32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _positions(kind, B, S):
    if kind == "arange":
        return None, np.broadcast_to(np.arange(S), (B, S))
    # per-sequence offsets (left-padded batches) and a negative start
    pos = np.arange(S)[None, :] + np.array([37 * b - 5 for b in range(B)])[:, None]
    return pos.astype(np.int32), pos


PRE_CASES = [
    # B, S, Hq, Hkv, D, causal, dtype, positions, theta, factor
    (1, 128, 8, 2, 64, True, "fp32", "arange", 1e4, 1.0),      # the tiny fp32 workload's shape
    (4, 128, 32, 32, 128, True, "bf16", "arange", 1e4, 1.0),   # the S=128 causal RoPE workload's shape
    (2, 300, 8, 2, 128, True, "bf16", "offsets", 1e4, 2.0),    # ragged tiles, shifted positions, factor 2
    (2, 77, 4, 4, 64, False, "bf16", "arange", 5e5, 1.0),      # non-causal, large theta
    (2, 70, 4, 2, 64, True, "fp32", "offsets", 1e4, 2.0),
    (1, 1024, 64, 8, 128, True, "bf16", "arange", 1e4, 1.0),   # GQA, 4-wave grid
    (2, 2048, 32, 32, 128, True, "bf16", "arange", 1e4, 1.0),  # 8-wave grid
    (1, 2100, 8, 1, 128, True, "bf16", "offsets", 1e4, 1.0),   # four key groups
]


@pytest.mark.parametrize("B,S,Hq,Hkv,D,causal,dtype,pk,theta,factor", PRE_CASES)
def test_rope_attn_prefill(B, S, Hq, Hkv, D, causal, dtype, pk, theta, factor):
    import torch
    announce(f"rope_attn_prefill B={B} S={S} Hq={Hq} Hkv={Hkv} D={D} causal={causal} {dtype} {pk}")
    seed = 11 + S + Hq + D
    q = W.random_case(seed, (B, S, Hq, D), dtype)
    k = W.random_case(seed + 1, (B, S, Hkv, D), dtype)
    v = W.random_case(seed + 2, (B, S, Hkv, D), dtype)
    pos_dev, pos = _positions(pk, B, S)
    pos_t = None if pos_dev is None else _i32(pos_dev)
    scale = D ** -0.5
    qd, kd, vd = dev(q, dtype), dev(k, dtype), dev(v, dtype)
    q0 = qd.clone()
    out = R.rope_attn_prefill(qd, kd, vd, pos_t, causal=causal, scale=scale, theta=theta, linear_factor=factor)
    # the separate calls on copies of the same inputs
    q2, k2 = dev(q, dtype), dev(k, dtype)
    R.rope_apply(q2, k2, pos_t, theta, factor)
    ref_gpu = R.attn_prefill(q2, k2, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(qd, q0), "q must not be modified"
    assert torch.equal(kd, k2), "k must be rotated in place exactly as rope_apply rotates it"
    assert torch.equal(out, ref_gpu), "fused result differs from rope_apply + attn_prefill"
    # against the oracle, every (batch, head) slice
    q64, k64, v64 = W.to_f64(q, dtype), W.to_f64(k, dtype), W.to_f64(v, dtype)
    ref, k_rot = oracle.rope_attention(q64, k64, v64, pos, causal, scale, theta, factor)
    check(host64(kd), k_rot, dtype, "rope_attn_prefill k")
    got = host64(out)
    for b in range(B):
        for h in range(Hq):
            check(got[b, :, h], ref[b, :, h], dtype, f"rope_attn_prefill b={b} h={h}")


def test_rope_attn_prefill_c3_bitwise():
    """The 7B-shaped workload: fused == separate calls, bit for bit."""
    import torch
    announce("rope_attn_prefill c3 bitwise")
    w = W.WORKLOADS["c3"]
    q, k, v = W.prefill_inputs(w)
    qd, kd, vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    q2, k2 = qd.clone(), kd.clone()
    out = R.rope_attn_prefill(qd, kd, vd, causal=True, scale=w.scale, theta=w.theta)
    R.rope_apply(q2, k2, None, w.theta)
    ref = R.attn_prefill(q2, k2, vd, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(kd, k2)
    assert torch.equal(out, ref)


def _decode_case(seed, B, Hq, Hkv, D, max_kv, dtype):
    q = W.random_case(seed, (B, Hq, D), dtype)
    kn = W.random_case(seed + 1, (B, Hkv, D), dtype)
    vn = W.random_case(seed + 2, (B, Hkv, D), dtype)
    kc = W.random_case(seed + 3, (B, Hkv, max_kv, D), dtype)
    vc = W.random_case(seed + 4, (B, Hkv, max_kv, D), dtype)
    return q, kn, vn, kc, vc


DEC_CASES = [
    # B, Hq, Hkv, D, max_kv, kv_lens, positions, factor, dtype
    (4, 32, 4, 128, 3000, [1, 513, 2048, 3000], None, 2.0, "bf16"),
    (3, 16, 2, 64, 700, [0, 700, 801], None, 1.0, "bf16"),          # empty sequence, row past the cache
    (2, 8, 8, 128, 300, [150, 299], [4000, 7], 1.0, "bf16"),        # explicit positions
    (2, 16, 1, 128, 400, [37, 400], None, 2.0, "fp32"),
]


@pytest.mark.parametrize("B,Hq,Hkv,D,max_kv,lens,pos,factor,dtype", DEC_CASES)
def test_rope_attn_decode(B, Hq, Hkv, D, max_kv, lens, pos, factor, dtype):
    import torch
    announce(f"rope_attn_decode B={B} Hq={Hq} Hkv={Hkv} D={D} lens={lens} pos={pos} {dtype}")
    seed = 300 + B + Hq + max_kv
    q, kn, vn, kc, vc = _decode_case(seed, B, Hq, Hkv, D, max_kv, dtype)
    scale, theta = D ** -0.5, 1e4
    lens_t = _i32(lens)
    pos_t = None if pos is None else _i32(pos)
    qd, knd, vnd = dev(q, dtype), dev(kn, dtype), dev(vn, dtype)
    kcd, vcd = dev(kc, dtype), dev(vc, dtype)
    out = R.rope_attn_decode(qd, knd, vnd, kcd, vcd, lens_t, pos_t, scale=scale, theta=theta, linear_factor=factor)
    # the separate calls on copies
    q2, kn2 = dev(q, dtype).view(B, 1, Hq, D), dev(kn, dtype).view(B, 1, Hkv, D)
    kc2, vc2 = dev(kc, dtype), dev(vc, dtype)
    p = np.array(lens) - 1 if pos is None else np.array(pos)
    R.rope_apply(q2, kn2, _i32(p.reshape(B, 1)), theta, factor)
    R.kv_append(kc2, vc2, kn2.view(B, Hkv, D), vnd, _i32(np.array(lens) - 1))
    ref_gpu = R.attn_decode(q2.view(B, Hq, D), kc2, vc2, lens_t, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(kcd, kc2) and torch.equal(vcd, vc2), "cache update differs from rope_apply + kv_append"
    assert torch.equal(out, ref_gpu), "fused result differs from the separate calls"
    ref, kc64, _ = oracle.rope_decode_step(W.to_f64(q, dtype), W.to_f64(kn, dtype), W.to_f64(vn, dtype),
                                           W.to_f64(kc, dtype), W.to_f64(vc, dtype), np.array(lens),
                                           None if pos is None else np.array(pos), scale, theta, factor)
    check(host64(out), ref, dtype, "rope_attn_decode out")
    for b, L in enumerate(lens):
        if 1 <= L <= max_kv:
            check(host64(kcd[b, :, L - 1]), kc64[b, :, L - 1], dtype, f"appended key b={b}")


def test_rope_attn_decode_c5_subset():
    """Sixteen sequences of the decode workload (factor 2, position = context)."""
    import torch
    w = W.WORKLOADS["c5"]
    announce("rope_attn_decode c5 B=16")
    inp = W.decode_inputs(w, B=16)
    B = 16
    ctx = inp["ctx"]
    qd, knd, vnd = dev(inp["q"], "bf16"), dev(inp["k_new"], "bf16"), dev(inp["v_new"], "bf16")
    kcd, vcd = dev(inp["k_cache"], "bf16"), dev(inp["v_cache"], "bf16")
    out = R.rope_attn_decode(qd, knd, vnd, kcd, vcd, _i32(ctx + 1), None, scale=w.scale, theta=w.theta,
                             linear_factor=w.factor)
    torch.cuda.synchronize()
    got = host64(out)
    del kcd, vcd
    ref = np.zeros((B, w.Hq, w.D))
    for b in range(B):   # one sequence at a time keeps the float64 cache small
        L = int(ctx[b]) + 1
        kc64 = W.to_f64(inp["k_cache"][b:b + 1, :, :L], "bf16")
        vc64 = W.to_f64(inp["v_cache"][b:b + 1, :, :L], "bf16")
        ref[b] = oracle.rope_decode_step(W.to_f64(inp["q"][b:b + 1], "bf16"), W.to_f64(inp["k_new"][b:b + 1], "bf16"),
                                         W.to_f64(inp["v_new"][b:b + 1], "bf16"), kc64, vc64, np.array([L]), None,
                                         w.scale, w.theta, w.factor)[0][0]
    check(got, ref, "bf16", "rope_attn_decode c5 subset")
