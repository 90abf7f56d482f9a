"""attn_decode_noalloc (split-K partial states in the library's fixed per-GPU
scratch) against attn_decode with a caller-owned workspace, through the C ABI.

The two entry points run the same kernels, so their outputs must be identical
bit for bit; the oracle comparison pins the no-allocation result to the parity
bars as well.  Calls come in a row with the second one smaller, so a result
that leaned on what an earlier call left in the scratch would show."""
import ctypes

import numpy as np
import pytest

import oracle
import rope_causal_gqa_amd as R
from rope_causal_gqa_amd import _binding as Bd
from rope_causal_gqa_amd import workloads as W
from tests.gpu_helpers import announce, check, dev, host64

pytestmark = pytest.mark.gpu


def _case(seed, B, Hq, Hkv, D, max_kv, lens, dtype):
    rng = np.random.Generator(np.random.PCG64(seed))
    q = W.draw(rng, (B, Hq, D), dtype)
    kc = W.draw(rng, (B, Hkv, max_kv, D), dtype)
    vc = W.draw(rng, (B, Hkv, max_kv, D), dtype)
    return q, kc, vc, np.asarray(lens, dtype=np.int32)


def _noalloc_c(qd, kcd, vcd, lens_d, outd, B, Hq, Hkv, D, max_kv, scale, dt):
    """The C symbol called directly (argument marshalling by hand)."""
    import torch
    L = Bd.lib()
    st = torch.cuda.current_stream().cuda_stream
    return L.attn_decode_noalloc(ctypes.c_void_p(qd.data_ptr()), ctypes.c_void_p(kcd.data_ptr()),
                                 ctypes.c_void_p(vcd.data_ptr()), ctypes.c_void_p(lens_d.data_ptr()),
                                 ctypes.c_void_p(outd.data_ptr()), B, Hq, Hkv, D, max_kv, float(scale), dt,
                                 ctypes.c_void_p(st))


def _run(seed, B, Hq, Hkv, D, max_kv, lens, dtype, oracle_rows=None):
    import torch
    announce(f"decode_noalloc seed={seed} B={B} Hq={Hq} Hkv={Hkv} D={D} max_kv={max_kv} {dtype}")
    q, kc, vc, lens = _case(seed, B, Hq, Hkv, D, max_kv, lens, dtype)
    qd, kcd, vcd = dev(q, dtype), dev(kc, dtype), dev(vc, dtype)
    lens_d = torch.from_numpy(lens).cuda()
    scale = D ** -0.5
    dt = Bd.BF16 if dtype == "bf16" else Bd.FP32
    ref_out = R.attn_decode(qd, kcd, vcd, lens_d, scale=scale)
    got = torch.full_like(ref_out, float("nan"))
    assert _noalloc_c(qd, kcd, vcd, lens_d, got, B, Hq, Hkv, D, max_kv, scale, dt) == Bd.OK
    torch.cuda.synchronize()
    assert torch.equal(got, ref_out), "attn_decode_noalloc differs from attn_decode"
    # and the binding reaches the same symbol
    got2 = R.attn_decode_noalloc(qd, kcd, vcd, lens_d, torch.empty_like(ref_out), scale)
    torch.cuda.synchronize()
    assert torch.equal(got2, ref_out)
    rows = range(B) if oracle_rows is None else oracle_rows
    got64 = host64(got)
    for b in rows:
        Lb = int(min(max(lens[b], 0), max_kv))
        ref = oracle.decode(W.to_f64(q[b:b + 1], dtype), W.to_f64(kc[b:b + 1, :, :max(Lb, 1)], dtype),
                            W.to_f64(vc[b:b + 1, :, :max(Lb, 1)], dtype), np.array([Lb]), scale)
        check(got64[b:b + 1], ref, dtype, f"decode_noalloc row {b}")


def test_noalloc_two_calls_second_smaller():
    # lengths at 0, 1, a split boundary (2048 keys) and either side of it, max_kv and past it
    _run(11, 8, 16, 2, 128, 3000, [0, 1, 2047, 2048, 2049, 3000, 5000, 1234], "bf16")
    _run(12, 3, 8, 1, 128, 500, [500, 17, 499], "bf16")


def test_noalloc_fp32_and_head_dim_64():
    _run(13, 4, 8, 2, 64, 700, [700, 256, 257, 3], "fp32")
    _run(14, 2, 4, 4, 64, 300, [300, 1], "fp32")


def test_noalloc_decode_workload_size():
    """The B=64 Hq=64 Hkv=8 D=128 decode against an 8193-row cache (10.6 MB of
    partial states); the caches are drawn on the device, and three sequences
    are checked against the oracle from host copies of their rows."""
    import torch
    w = W.WORKLOADS["c5"]
    announce("decode_noalloc B=64 Hq=64 Hkv=8 D=128 max_kv=8193 bf16")
    rng = np.random.Generator(np.random.PCG64(w.seed))
    lens = (rng.integers(w.ctx_lo, w.ctx_hi + 1, size=w.B) + 1).astype(np.int32)
    g = torch.Generator(device="cuda")
    g.manual_seed(w.seed)
    qd = torch.randn((w.B, w.Hq, w.D), generator=g, device="cuda").to(torch.bfloat16)
    kcd = torch.randn((w.B, w.Hkv, w.max_kv, w.D), generator=g, device="cuda").to(torch.bfloat16)
    vcd = torch.randn((w.B, w.Hkv, w.max_kv, w.D), generator=g, device="cuda").to(torch.bfloat16)
    lens_d = torch.from_numpy(lens).cuda()
    ref_out = R.attn_decode(qd, kcd, vcd, lens_d, scale=w.scale)
    got = torch.full_like(ref_out, float("nan"))
    assert _noalloc_c(qd, kcd, vcd, lens_d, got, w.B, w.Hq, w.Hkv, w.D, w.max_kv, w.scale, Bd.BF16) == Bd.OK
    torch.cuda.synchronize()
    assert torch.equal(got, ref_out), "attn_decode_noalloc differs from attn_decode"
    got64 = host64(got)
    for b in (0, 31, 63):
        L = int(lens[b])
        ref = oracle.decode(host64(qd[b:b + 1]), host64(kcd[b:b + 1, :, :L]), host64(vcd[b:b + 1, :, :L]),
                            np.array([L]), w.scale)
        check(got64[b:b + 1], ref, "bf16", f"decode_noalloc c5 row {b}")
    del kcd, vcd
    # then a smaller call again
    _run(16, 2, 8, 8, 128, 100, [100, 50], "bf16")


def test_noalloc_rejects_oversize_before_launch():
    import torch
    # 64 * 64 * ceil(16385 / 2048) * 130 * 4 bytes > 16 MiB; the check precedes any launch,
    # so small buffers with the large declared sizes are never touched
    small = torch.zeros(64 * 64 * 128, dtype=torch.bfloat16, device="cuda")
    out = torch.zeros_like(small)
    lens = torch.ones(64, dtype=torch.int32, device="cuda")
    st = _noalloc_c(small, small, small, lens, out, 64, 64, 8, 128, 16385, 128 ** -0.5, Bd.BF16)
    assert st == Bd.ENOSPACE
    assert b"scratch" in Bd.lib().rcgqa_status_string(st)
    torch.cuda.synchronize()
