"""attn_decode / kv_append (and the rope -> append -> decode path) on the GPU
against the float64 oracle."""
import math

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


def _decode_path(w, inp):
    """GPU: rope q/k_new at pos=ctx (factor) -> append at slot ctx -> decode with kv_len = ctx + 1.
    Oracle: the same steps in float64.  Returns (got, ref) [B, Hq, D]."""
    import torch
    B = inp["ctx"].shape[0]
    ctx = inp["ctx"]
    dt = w.dtype
    qd = dev(inp["q"], dt).view(B, 1, w.Hq, w.D)
    knd = dev(inp["k_new"], dt).view(B, 1, w.Hkv, w.D)
    vnd = dev(inp["v_new"], dt)
    kc, vc = dev(inp["k_cache"], dt), dev(inp["v_cache"], dt)
    R.rope_apply(qd, knd, _i32(ctx.reshape(B, 1)), w.theta, w.factor)
    R.kv_append(kc, vc, knd.view(B, w.Hkv, w.D), vnd, _i32(ctx))
    out = R.attn_decode(qd.view(B, w.Hq, w.D), kc, vc, _i32(ctx + 1), scale=w.scale)
    torch.cuda.synchronize()
    got = host64(out)
    del kc, vc
    q64 = W.to_f64(inp["q"], dt).reshape(B, 1, w.Hq, w.D)
    kn64 = W.to_f64(inp["k_new"], dt).reshape(B, 1, w.Hkv, w.D)
    qr, knr = oracle.rope_apply(q64, kn64, ctx.reshape(B, 1), w.theta, w.factor)
    ref = np.zeros((B, w.Hq, w.D))
    for b in range(B):   # one sequence at a time keeps the float64 cache small
        L = int(ctx[b]) + 1
        kc64 = W.to_f64(inp["k_cache"][b:b + 1, :, :L], dt)
        vc64 = W.to_f64(inp["v_cache"][b:b + 1, :, :L], dt)
        kc64, vc64 = oracle.kv_append(kc64, vc64, knr[b:b + 1, 0], W.to_f64(inp["v_new"][b:b + 1], dt),
                                      np.array([L - 1]))
        ref[b] = oracle.decode(qr[b:b + 1, 0], kc64, vc64, np.array([L]), w.scale)[0]
    return got, ref


def test_decode_c5_full():
    w = W.WORKLOADS["c5"]
    announce("decode c5 full B=64")
    got, ref = _decode_path(w, W.decode_inputs(w))
    check(got, ref, "bf16", "rope+append+decode c5")


DEC_EDGE = [
    # B, Hq, Hkv, D, max_kv, lens, dtype
    (4, 8, 1, 128, 600, [1, 255, 256, 257], "bf16"),
    (3, 16, 8, 128, 1025, [1024, 1025, 513], "bf16"),
    (2, 8, 8, 64, 700, [700, 2], "bf16"),
    (2, 16, 1, 128, 300, [0, 1000], "bf16"),          # empty row and clamped length
    (3, 16, 1, 128, 300, [-5, 299, 0], "bf16"),       # negative length: an empty cache
    (5, 32, 2, 128, 2049, [2049, 7, 1536, 100, 1], "bf16"),
    (2, 8, 1, 128, 20000, [20000, 6145], "bf16"),     # > 8 splits: merge batches
    (2, 16, 1, 128, 4096, [4096, 2048], "bf16"),      # exact split multiples
    (2, 8, 2, 64, 400, [399, 1], "fp32"),
    (3, 4, 4, 128, 513, [513, 256, 0], "fp32"),
]


@pytest.mark.parametrize("B,Hq,Hkv,D,max_kv,lens,dtype", DEC_EDGE)
def test_decode_edges(B, Hq, Hkv, D, max_kv, lens, dtype):
    import torch
    announce(f"decode edge B={B} Hq={Hq} Hkv={Hkv} D={D} max_kv={max_kv} lens={lens} {dtype}")
    seed = B * 31 + Hq * 7 + max_kv
    q = W.random_case(seed, (B, Hq, D), dtype)
    kc = W.random_case(seed + 1, (B, Hkv, max_kv, D), dtype)
    vc = W.random_case(seed + 2, (B, Hkv, max_kv, D), dtype)
    lens = np.array(lens, dtype=np.int32)
    scale = 1.0 / math.sqrt(D)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    n = B * Hq * D
    buf = torch.full((n + 2048,), 7.0, dtype=tdt, device="cuda")
    out = buf[1024:1024 + n].view(B, Hq, D)
    R.attn_decode(dev(q, dtype), dev(kc, dtype), dev(vc, dtype), _i32(lens), out, scale=scale)
    torch.cuda.synchronize()
    assert torch.all(buf[:1024] == 7.0) and torch.all(buf[1024 + n:] == 7.0), "write outside out"
    ref = oracle.decode(W.to_f64(q, dtype), W.to_f64(kc, dtype), W.to_f64(vc, dtype), lens, scale)
    check(host64(out), ref, dtype, f"decode edge lens={lens.tolist()}")
    for b, L in enumerate(lens):
        if L <= 0:
            assert np.all(host64(out)[b] == 0.0)


def test_decode_deterministic_and_workspace_reuse():
    import torch
    B, Hq, Hkv, D, max_kv = 4, 16, 2, 128, 3000
    q = dev(W.random_case(1, (B, Hq, D), "bf16"), "bf16")
    kc = dev(W.random_case(2, (B, Hkv, max_kv, D), "bf16"), "bf16")
    vc = dev(W.random_case(3, (B, Hkv, max_kv, D), "bf16"), "bf16")
    lens = _i32([3000, 1, 2048, 777])
    ws = torch.full((R.attn_decode_workspace_bytes(B, Hq, D, max_kv),), 255, dtype=torch.uint8, device="cuda")
    a = R.attn_decode(q, kc, vc, lens, scale=D ** -0.5, workspace=ws)
    b = R.attn_decode(q, kc, vc, lens, scale=D ** -0.5, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_kv_append_rows():
    import torch
    B, Hkv, D, max_kv = 3, 2, 64, 10
    kc = dev(W.random_case(1, (B, Hkv, max_kv, D), "bf16"), "bf16")
    vc = dev(W.random_case(2, (B, Hkv, max_kv, D), "bf16"), "bf16")
    kn = dev(W.random_case(3, (B, Hkv, D), "bf16"), "bf16")
    vn = dev(W.random_case(4, (B, Hkv, D), "bf16"), "bf16")
    k0, v0 = kc.clone(), vc.clone()
    slots = np.array([0, 9, 10], dtype=np.int32)     # last one is out of range: no write
    R.kv_append(kc, vc, kn, vn, _i32(slots))
    torch.cuda.synchronize()
    rk, rv = oracle.kv_append(host64(k0), host64(v0), host64(kn), host64(vn), slots)
    assert np.array_equal(host64(kc), rk) and np.array_equal(host64(vc), rv)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_decode_growing_scores(dtype):
    """Cache keys whose scores grow with their position: every split of the
    split-K pass (and the merge) sees maxima far apart."""
    import torch
    announce(f"decode growing scores {dtype}")
    B, Hq, Hkv, D, max_kv = 3, 16, 2, 128, 5000
    r = np.random.Generator(np.random.PCG64(404))
    u = r.standard_normal(D)
    u /= np.linalg.norm(u)
    # fp32 keeps scores within ~20 so its rounding (proportional to |score|) stays under 1e-5
    q = (30.0 if dtype == "bf16" else 10.0) * u + 0.3 * r.standard_normal((B, Hq, D))
    kc = (np.arange(max_kv) / (200.0 if dtype == "bf16" else 400.0))[None, None, :, None] * u + 0.3 * r.standard_normal((B, Hkv, max_kv, D))
    vc = r.standard_normal((B, Hkv, max_kv, D))
    lens = np.array([4999, 2500, 700])
    if dtype == "bf16":
        q, kc, vc = (W.round_bf16(a) for a in (q, kc, vc))
    else:
        q, kc, vc = (a.astype(np.float32) for a in (q, kc, vc))
    out = R.attn_decode(dev(q, dtype), dev(kc, dtype), dev(vc, dtype), _i32(lens), scale=D ** -0.5)
    torch.cuda.synchronize()
    ref = oracle.decode(W.to_f64(q, dtype), W.to_f64(kc, dtype), W.to_f64(vc, dtype), lens, D ** -0.5)
    check(host64(out), ref, dtype, f"decode growing scores {dtype}")
