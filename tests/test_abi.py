"""The C-ABI library loads and exports what include/rcgqa.h declares; host-side
argument checks reject bad calls before any launch (CPU only: no call here
passes validation, so nothing reaches the GPU)."""
import ctypes
import os
import re

import pytest

import rope_causal_gqa_amd as R
from rope_causal_gqa_amd import _binding as BD

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "rcgqa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(R.lib_path()), reason="librcgqa.so not built")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", src)) - {"if", "sizeof"})


def test_exports_every_declared_symbol():
    names = _declared()
    assert set(names) >= {"rope_apply", "rope_apply_interleaved", "attn_prefill", "attn_prefill_cache", "attn_decode",
                          "attn_decode_workspace_bytes", "kv_append", "rcgqa_status_string"}
    L = R.lib()
    for n in names:
        assert hasattr(L, n), n
    out = os.popen(f"nm -D --defined-only {R.lib_path()}").read()
    for n in names:
        assert re.search(rf"\sT {n}$", out, re.M), n


def test_status_strings():
    L = R.lib()
    assert L.rcgqa_status_string(0) == b"ok"
    assert L.rcgqa_status_string(1) == b"invalid argument"
    assert L.rcgqa_status_string(2).startswith(b"unsupported")
    assert L.rcgqa_status_string(3).startswith(b"HIP")
    assert b"scratch" in L.rcgqa_status_string(4)
    assert L.rcgqa_status_string(99) == b"unknown status"


def test_workspace_bytes():
    L = R.lib()
    a = L.attn_decode_workspace_bytes(64, 64, 128, 8193)
    assert a >= 64 * 64 * 130 * 4                  # at least one partial state per row
    assert L.attn_decode_workspace_bytes(64, 64, 128, 16386) >= a
    assert L.attn_decode_workspace_bytes(0, 64, 128, 10) == 0
    assert L.attn_decode_workspace_bytes(1, 1, 128, -1) == 0


FAKE = ctypes.c_void_p(4096)   # never dereferenced: every call below fails validation


@pytest.mark.parametrize("args", [
    dict(q=None),
    dict(B=0), dict(S=0), dict(Hq=0), dict(Hkv=0), dict(Hq=6, Hkv=4),
    dict(D=63), dict(D=0), dict(theta=0.0), dict(theta=float("inf")), dict(factor=0.0),
    dict(factor=float("nan")), dict(dt=7),
])
@pytest.mark.parametrize("name", ["rope_apply", "rope_apply_interleaved"])
def test_rope_rejects(args, name):
    a = dict(q=FAKE, k=FAKE, B=1, S=4, Hq=8, Hkv=2, D=64, theta=1e4, factor=1.0, dt=0)
    a.update(args)
    st = getattr(R.lib(), name)(a["q"], a["k"], None, a["B"], a["S"], a["Hq"], a["Hkv"], a["D"], a["theta"],
                                a["factor"], a["dt"], None)
    assert st == BD.EINVAL


@pytest.mark.parametrize("name", ["rope_apply", "rope_apply_interleaved"])
def test_rope_unsupported_head_dim(name):
    assert getattr(R.lib(), name)(FAKE, FAKE, None, 1, 1, 1, 1, 258, 1e4, 1.0, 0, None) == BD.EUNSUPPORTED


@pytest.mark.parametrize("args", [
    dict(out=None), dict(same=True), dict(B=-1), dict(Hq=3, Hkv=2), dict(causal=2), dict(scale=0.0),
    dict(scale=float("nan")), dict(D=7),
])
def test_prefill_rejects(args):
    a = dict(q=FAKE, out=ctypes.c_void_p(8192), B=1, S=4, Hq=8, Hkv=2, D=64, causal=1, scale=0.125, dt=0)
    a.update(args)
    out = a["q"] if a.get("same") else a["out"]
    st = R.lib().attn_prefill(a["q"], FAKE, FAKE, out, a["B"], a["S"], a["Hq"], a["Hkv"], a["D"], a["causal"],
                              a["scale"], a["dt"], None)
    assert st == BD.EINVAL


@pytest.mark.parametrize("D", [32, 96, 256])
def test_prefill_unsupported_head_dim(D):
    assert R.lib().attn_prefill(FAKE, FAKE, FAKE, ctypes.c_void_p(8192), 1, 4, 8, 2, D, 1, 0.1, 0, None) \
        == BD.EUNSUPPORTED


@pytest.mark.parametrize("args", [
    dict(out=None), dict(same=True), dict(lens=None), dict(B=0), dict(Sq=0), dict(Hq=6, Hkv=4),
    dict(max_kv=0), dict(D=5), dict(causal=3), dict(window=-1), dict(window=8, causal=0), dict(scale=0.0),
    dict(scale=float("inf")), dict(dt=5),
])
def test_prefill_cache_rejects(args):
    a = dict(q=FAKE, out=ctypes.c_void_p(8192), lens=FAKE, B=2, Sq=16, Hq=8, Hkv=2, D=128, max_kv=100, causal=1,
             window=0, scale=0.1, dt=0)
    a.update(args)
    out = a["q"] if a.get("same") else a["out"]
    st = R.lib().attn_prefill_cache(a["q"], FAKE, FAKE, a["lens"], out, a["B"], a["Sq"], a["Hq"], a["Hkv"], a["D"],
                                    a["max_kv"], a["causal"], a["window"], a["scale"], a["dt"], None)
    assert st == BD.EINVAL


def test_prefill_cache_workspace_bytes():
    L = R.lib()
    # a chunk of 512 new tokens after 4096 cached ones, 16 heads x 2 sequences: stream-K, 256 workgroups
    assert L.attn_prefill_cache_workspace_bytes(2, 512, 16, 128, 4608, 1, 0) == 4096 + 256 * 2 * 256 * (2 * 128 + 16)
    assert L.attn_prefill_cache_workspace_bytes(2, 512, 16, 128, 4608, 1, 1024) == 0   # windowed
    assert L.attn_prefill_cache_workspace_bytes(2, 512, 16, 128, 4608, 1, 4608) > 0    # a window of max_kv is none
    assert L.attn_prefill_cache_workspace_bytes(2, 512, 16, 128, 4608, 0, 0) == 0      # not causal
    assert L.attn_prefill_cache_workspace_bytes(2, 512, 16, 128, 400, 1, 0) == 0       # cache shorter than the chunk
    assert L.attn_prefill_cache_workspace_bytes(2, 512, 32, 128, 4608, 1, 0) == 0      # the key-group grid is full
    assert L.attn_prefill_cache_workspace_bytes(64, 512, 32, 128, 4608, 1, 0) == 0     # paired grid
    assert L.attn_prefill_cache_workspace_bytes(1, 512, 8, 128, 4096, 1, 0) == 0       # too little work
    assert L.attn_prefill_cache_workspace_bytes(0, 512, 8, 128, 4096, 1, 0) == 0
    assert L.attn_prefill_cache_workspace_bytes(2, 512, 16, 128, 4608, 1, -1) == 0
    # a chunk that is the whole sequence plans as the plain prefill
    assert L.attn_prefill_cache_workspace_bytes(1, 8192, 2, 128, 8192, 1, 0) == L.attn_prefill_workspace_bytes(1, 8192, 2, 128, 1) > 0


@pytest.mark.parametrize("args", [
    dict(ws=None), dict(wbytes=100), dict(ws_addr=4096 * 64 + 64), dict(ws_is="out"), dict(ws_is="lens"),
    dict(lens=None), dict(Hq=6, Hkv=4), dict(window=-1), dict(window=8, causal=0), dict(max_kv=0), dict(causal=2),
    dict(scale=0.0), dict(dt=3),
])
def test_prefill_cache_ws_rejects(args):
    a = dict(B=2, Sq=512, Hq=16, Hkv=16, D=128, max_kv=4608, causal=1, window=0, scale=0.1, dt=0, ws_addr=4096 * 64,
             wbytes=1 << 30, lens=A[4])
    a.update(args)
    q, kc, vc, out = A[0], A[1], A[2], A[3]
    ws = ctypes.c_void_p(a["ws_addr"])
    if "ws" in args:
        ws = None
    elif args.get("ws_is") == "out":
        ws = out
    elif args.get("ws_is") == "lens":
        ws = a["lens"]
    st = R.lib().attn_prefill_cache_ws(q, kc, vc, a["lens"], out, a["B"], a["Sq"], a["Hq"], a["Hkv"], a["D"],
                                       a["max_kv"], a["causal"], a["window"], a["scale"], a["dt"], ws, a["wbytes"],
                                       None)
    assert st == BD.EINVAL


def test_prefill_cache_unsupported_head_dim():
    assert R.lib().attn_prefill_cache(FAKE, FAKE, FAKE, FAKE, ctypes.c_void_p(8192), 1, 4, 8, 2, 96, 10, 1, 0, 0.1,
                                      0, None) == BD.EUNSUPPORTED


@pytest.mark.parametrize("args", [
    dict(ws=None), dict(wbytes=0), dict(ws_addr=4096 + 8), dict(Hq=12, Hkv=8), dict(max_kv=0), dict(scale=-1.0),
    dict(lens=None),
])
def test_decode_rejects(args):
    a = dict(B=2, Hq=8, Hkv=2, D=128, max_kv=300, scale=0.1, ws_addr=4096 * 16, wbytes=1 << 30, lens=FAKE)
    a.update(args)
    ws = None if "ws" in args else ctypes.c_void_p(a["ws_addr"])
    st = R.lib().attn_decode(FAKE, FAKE, FAKE, a["lens"], ctypes.c_void_p(8192), a["B"], a["Hq"], a["Hkv"], a["D"],
                             a["max_kv"], a["scale"], 0, ws, a["wbytes"], None)
    assert st == BD.EINVAL


def test_decode_rejects_aliased_output():
    ws = ctypes.c_void_p(4096 * 16)
    q, k, v = (ctypes.c_void_p(4096 * i) for i in (3, 4, 5))
    for out in (q, k, v):
        assert R.lib().attn_decode(q, k, v, FAKE, out, 1, 8, 2, 128, 10, 0.1, 0, ws, 1 << 30, None) == BD.EINVAL
        assert R.lib().attn_decode_noalloc(q, k, v, FAKE, out, 1, 8, 2, 128, 10, 0.1, 0, None) == BD.EINVAL


@pytest.mark.parametrize("args", [
    dict(Hq=12, Hkv=8), dict(max_kv=0), dict(scale=-1.0), dict(scale=float("nan")), dict(lens=None), dict(D=63),
    dict(B=0), dict(dt=7),
])
def test_decode_noalloc_rejects(args):
    a = dict(B=2, Hq=8, Hkv=2, D=128, max_kv=300, scale=0.1, lens=FAKE, dt=0)
    a.update(args)
    st = R.lib().attn_decode_noalloc(FAKE, FAKE, FAKE, a["lens"], ctypes.c_void_p(8192), a["B"], a["Hq"], a["Hkv"],
                                     a["D"], a["max_kv"], a["scale"], a["dt"], None)
    assert st == BD.EINVAL


@pytest.mark.parametrize("B,Hq,D,max_kv,dt,fits", [
    (64, 64, 128, 8193, 0, True),     # the B=64 Hq=64 decode workload: 10.6 MB of partial states
    (64, 64, 128, 14336, 0, True),    # 7 splits of 2048 keys: 14.9 MB
    (64, 64, 128, 16385, 0, False),   # 9 splits: 19.2 MB > 16 MiB
    (64, 64, 128, 1792, 1, True),     # fp32 keeps a partial state per 256 keys: 7 of them, 14.9 MB
    (64, 64, 128, 2048, 1, False),    # 8 fp32 partial states: 17.0 MB
])
def test_decode_noalloc_limit(B, Hq, D, max_kv, dt, fits):
    """The size rule of the fixed scratch, checked on the host before any launch."""
    per = 2048 if dt == 0 else 256
    need = B * Hq * (-(-max_kv // per)) * (D + 2) * 4
    assert (need <= 16 << 20) == fits
    if not fits:
        st = R.lib().attn_decode_noalloc(FAKE, FAKE, FAKE, FAKE, ctypes.c_void_p(8192), B, Hq, 8, D, max_kv, 0.1, dt,
                                         None)
        assert st == BD.ENOSPACE


def test_decode_unsupported_group():
    st = R.lib().attn_decode(FAKE, FAKE, FAKE, FAKE, ctypes.c_void_p(8192), 1, 32, 1, 128, 10, 0.1, 0,
                             ctypes.c_void_p(4096 * 16), 1 << 30, None)
    assert st == BD.EUNSUPPORTED


@pytest.mark.parametrize("B,S,Hq,Hkv", [
    (1, 65535 * 64 + 1, 8, 2),     # more than 65535 64-row blocks in one sequence
    (1 << 16, 1, 512, 512),        # 2^25 (batch, head) pairs x 256 work-items > 2^32
    (1 << 12, 2049, 256, 256),     # 2^20 pairs x 17 row blocks of 128 x 256 > 2^32
])
def test_prefill_grid_limits(B, S, Hq, Hkv):
    L = R.lib()
    O = ctypes.c_void_p(8192)
    assert L.attn_prefill(FAKE, FAKE, FAKE, O, B, S, Hq, Hkv, 64, 1, 0.1, 0, None) == BD.EUNSUPPORTED
    assert L.attn_prefill_masked(FAKE, FAKE, FAKE, FAKE, O, B, S, Hq, Hkv, 64, 1, S, 1, 0.1, 0, None) \
        == BD.EUNSUPPORTED
    assert L.attn_prefill_cache(FAKE, FAKE, FAKE, FAKE, O, B, S, Hq, Hkv, 64, S, 1, 0, 0.1, 0, None) \
        == BD.EUNSUPPORTED
    q, k, v = (ctypes.c_void_p(4096 * i) for i in (3, 4, 5))
    assert L.rope_attn_prefill(q, k, v, O, None, B, S, Hq, Hkv, 64, 1, 0.1, 1e4, 1.0, 0, FAKE, 1 << 62,
                               None) == BD.EUNSUPPORTED


@pytest.mark.parametrize("B,Hq,Hkv", [(65536, 8, 2), (2, 65536 * 2, 65536)])
def test_decode_grid_limits(B, Hq, Hkv):
    L = R.lib()
    ws = ctypes.c_void_p(4096 * 16)
    assert L.attn_decode(FAKE, FAKE, FAKE, FAKE, ctypes.c_void_p(8192), B, Hq, Hkv, 128, 16, 0.1, 0, ws, 1 << 62,
                         None) == BD.EUNSUPPORTED
    assert L.rope_attn_decode(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, ctypes.c_void_p(8192), B, Hq, Hkv, 128, 16,
                              0.1, 1e4, 1.0, 0, ws, 1 << 62, None) == BD.EUNSUPPORTED
    assert L.kv_append(FAKE, FAKE, FAKE, FAKE, FAKE, B, min(Hkv, 65536), 64, 4, 0, None) == BD.EUNSUPPORTED


def test_kv_append_rejects():
    L = R.lib()
    assert L.kv_append(FAKE, FAKE, FAKE, FAKE, None, 1, 1, 64, 4, 0, None) == BD.EINVAL
    assert L.kv_append(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 63, 4, 0, None) == BD.EINVAL
    assert L.kv_append(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 0, 0, None) == BD.EINVAL


MIS = ctypes.c_void_p(4096 + 2)   # not 16-byte (nor 4-byte) aligned
A = [ctypes.c_void_p(4096 * i) for i in range(1, 9)]
WS = ctypes.c_void_p(4096 * 64)


@pytest.mark.parametrize("call", [
    lambda L: L.rope_apply(MIS, A[1], None, 1, 4, 8, 2, 64, 1e4, 1.0, 0, None),
    lambda L: L.rope_apply_interleaved(A[0], MIS, None, 1, 4, 8, 2, 64, 1e4, 1.0, 0, None),
    lambda L: L.rope_apply(A[0], A[1], MIS, 1, 4, 8, 2, 64, 1e4, 1.0, 0, None),
    lambda L: L.attn_prefill(A[0], A[1], MIS, A[3], 1, 4, 8, 2, 64, 1, 0.125, 0, None),
    lambda L: L.attn_prefill_cache(A[0], A[1], A[2], MIS, A[4], 1, 4, 8, 2, 64, 16, 1, 0, 0.125, 0, None),
    lambda L: L.attn_prefill_masked(A[0], A[1], A[2], MIS, A[4], 1, 4, 8, 2, 64, 1, 4, 1, 0.125, 0, None),
    lambda L: L.attn_prefill_ws(A[0], MIS, A[2], A[3], 1, 4, 8, 2, 64, 1, 0.125, 0, WS, 1 << 20, None),
    lambda L: L.attn_prefill_cache_ws(A[0], A[1], A[2], MIS, A[4], 1, 4, 8, 2, 64, 16, 1, 0, 0.125, 0, WS, 1 << 20,
                                      None),
    lambda L: L.attn_decode(A[0], MIS, A[2], A[3], A[4], 1, 8, 2, 128, 16, 0.1, 0, WS, 1 << 30, None),
    lambda L: L.rope_attn_prefill(A[0], A[1], A[2], MIS, None, 1, 16, 8, 2, 64, 1, 0.125, 1e4, 1.0, 0, WS, 1 << 20,
                                  None),
    lambda L: L.rope_attn_decode(A[0], A[1], MIS, A[3], A[4], A[5], None, A[6], 1, 8, 2, 128, 16, 0.1, 1e4, 1.0, 0,
                                 WS, 1 << 30, None),
    lambda L: L.kv_append(A[0], A[1], MIS, A[3], A[4], 1, 2, 64, 16, 0, None),
])
def test_misaligned_pointers_rejected(call):
    assert call(R.lib()) == BD.EINVAL


def test_binding_requires_device_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 4, 2, 64)
    with pytest.raises(ValueError):
        R.rope_apply(q, q.clone())
    with pytest.raises(ValueError):
        R.attn_prefill(q, q, q, scale=0.125)
    with pytest.raises(ValueError):
        R.attn_prefill_cache(q, q, q, torch.zeros(1, dtype=torch.int32), scale=0.125)


def test_prefill_workspace_bytes():
    L = R.lib()
    # one GPU's 8-query-head share at 4096 tokens: stream-K over 256 workgroups,
    # 4 KB of counters, then two partial states per workgroup: 256 rows x D fp16, 256 x 4 floats
    n = L.attn_prefill_workspace_bytes(1, 4096, 8, 128, 1)
    assert n == 4096 + 256 * 2 * 256 * (2 * 128 + 16)
    assert L.attn_prefill_workspace_bytes(1, 4096, 8, 64, 1) < n
    assert L.attn_prefill_workspace_bytes(1, 4096, 8, 128, 0) == 0     # non-causal: no split
    assert L.attn_prefill_workspace_bytes(2, 4096, 64, 128, 1) == 0    # fills the GPU without one
    assert L.attn_prefill_workspace_bytes(1, 4096, 32, 128, 1) == 0    # paired 4-wave grid
    assert L.attn_prefill_workspace_bytes(1, 2100, 8, 128, 1) == 0     # too little work per workgroup
    assert L.attn_prefill_workspace_bytes(1, 16384, 4, 128, 1) == n    # long: 256 workgroups too
    assert L.attn_prefill_workspace_bytes(1, 32769, 2, 128, 1) == 0    # more than 128 query tiles
    assert L.attn_prefill_workspace_bytes(0, 4096, 8, 128, 1) == 0
    assert L.attn_prefill_workspace_bytes(1, 4096, 8, 96, 1) == 0


@pytest.mark.parametrize("args", [
    dict(ws=None), dict(wbytes=100), dict(ws_addr=4096 * 64 + 64), dict(ws_is_out=True), dict(out_is_q=True),
    dict(Hq=6, Hkv=4), dict(causal=2), dict(scale=0.0), dict(D=9), dict(dt=3),
])
def test_prefill_ws_rejects(args):
    a = dict(B=1, S=4096, Hq=8, Hkv=1, D=128, causal=1, scale=0.125, dt=0, ws_addr=4096 * 64, wbytes=1 << 30)
    a.update(args)
    q, k, v, out = A[0], A[1], A[2], A[3]
    if args.get("out_is_q"):
        out = q
    ws = None if "ws" in args else (out if args.get("ws_is_out") else ctypes.c_void_p(a["ws_addr"]))
    st = R.lib().attn_prefill_ws(q, k, v, out, a["B"], a["S"], a["Hq"], a["Hkv"], a["D"], a["causal"], a["scale"],
                                 a["dt"], ws, a["wbytes"], None)
    assert st == BD.EINVAL


def test_prefill_ws_unsupported_head_dim():
    assert R.lib().attn_prefill_ws(A[0], A[1], A[2], A[3], 1, 64, 8, 1, 96, 1, 0.1, 0, WS, 1 << 20, None) \
        == BD.EUNSUPPORTED


def test_fused_workspace_bytes():
    L = R.lib()
    assert L.rope_attn_prefill_workspace_bytes(2, 4096, 128) == 2 * 4096 * 128 * 4
    assert L.rope_attn_prefill_workspace_bytes(0, 4096, 128) == 0
    d = L.rope_attn_decode_workspace_bytes(64, 64, 128, 8193)
    assert d >= L.attn_decode_workspace_bytes(64, 64, 128, 8193) + 64 * 64 * 128 * 4
    assert L.rope_attn_decode_workspace_bytes(1, 0, 128, 10) == 0


@pytest.mark.parametrize("args", [
    dict(ws=None), dict(wbytes=100), dict(ws_addr=4096 + 64), dict(q_is_k=True), dict(k_is_v=True),
    dict(out_is_q=True), dict(Hq=6, Hkv=4), dict(theta=0.0), dict(factor=float("inf")), dict(causal=3),
    dict(scale=0.0), dict(D=9),
])
def test_rope_attn_prefill_rejects(args):
    a = dict(B=1, S=16, Hq=8, Hkv=2, D=64, causal=1, scale=0.125, theta=1e4, factor=1.0, ws_addr=4096 * 16,
             wbytes=1 << 20)
    a.update(args)
    q, k, v, out = ctypes.c_void_p(4096), ctypes.c_void_p(8192), ctypes.c_void_p(12288), ctypes.c_void_p(16384)
    if args.get("q_is_k"):
        k = q
    if args.get("k_is_v"):
        v = k
    if args.get("out_is_q"):
        out = q
    ws = None if "ws" in args else ctypes.c_void_p(a["ws_addr"])
    st = R.lib().rope_attn_prefill(q, k, v, out, None, a["B"], a["S"], a["Hq"], a["Hkv"], a["D"], a["causal"],
                                   a["scale"], a["theta"], a["factor"], 0, ws, a["wbytes"], None)
    assert st == BD.EINVAL


def test_rope_attn_prefill_unsupported_head_dim():
    st = R.lib().rope_attn_prefill(FAKE, ctypes.c_void_p(8192), ctypes.c_void_p(12288), ctypes.c_void_p(16384),
                                   None, 1, 16, 2, 2, 96, 1, 0.1, 1e4, 1.0, 0, ctypes.c_void_p(4096 * 16), 1 << 20,
                                   None)
    assert st == BD.EUNSUPPORTED


@pytest.mark.parametrize("args", [
    dict(ws=None), dict(wbytes=0), dict(ws_addr=4096 + 8), dict(lens=None), dict(Hq=12, Hkv=8), dict(max_kv=0),
    dict(theta=-1.0), dict(factor=0.0), dict(scale=float("nan")),
])
def test_rope_attn_decode_rejects(args):
    a = dict(B=2, Hq=8, Hkv=2, D=128, max_kv=300, scale=0.1, theta=1e4, factor=2.0, ws_addr=4096 * 16,
             wbytes=1 << 30, lens=FAKE)
    a.update(args)
    ws = None if "ws" in args else ctypes.c_void_p(a["ws_addr"])
    st = R.lib().rope_attn_decode(FAKE, FAKE, FAKE, FAKE, FAKE, a["lens"], None, ctypes.c_void_p(8192), a["B"],
                                  a["Hq"], a["Hkv"], a["D"], a["max_kv"], a["scale"], a["theta"], a["factor"], 0, ws,
                                  a["wbytes"], None)
    assert st == BD.EINVAL


def test_fused_binding_requires_device_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 4, 2, 64)
    with pytest.raises(ValueError):
        R.rope_attn_prefill(q, q.clone(), q.clone(), scale=0.125)
    with pytest.raises(ValueError):
        R.rope_attn_decode(torch.zeros(1, 2, 64), torch.zeros(1, 1, 64), torch.zeros(1, 1, 64),
                           torch.zeros(1, 1, 8, 64), torch.zeros(1, 1, 8, 64), torch.ones(1, dtype=torch.int32),
                           scale=0.125)


@pytest.mark.parametrize("theta,D,alpha", [(1e4, 128, 8.0), (5e5, 64, 2.5), (1e4, 4, 4.0), (100.0, 256, 0.5),
                                           (1e4, 128, 1.0)])
def test_ntk_theta_matches_oracle(theta, D, alpha):
    """Host-side arithmetic (nothing launched): the library's base against the
    oracle's float64 one, to float rounding."""
    import oracle
    assert R.rope_ntk_theta(theta, D, alpha) == pytest.approx(oracle.ntk_theta(theta, D, alpha), rel=2 ** -23)


@pytest.mark.parametrize("theta,D,f,L,L0", [(1e4, 128, 2.0, 8192, 4096), (1e4, 128, 2.0, 4096, 4096),
                                            (1e4, 64, 4.0, 5000, 2048), (5e5, 128, 1.0, 100, 4096)])
def test_dynamic_ntk_theta_matches_oracle(theta, D, f, L, L0):
    import oracle
    got = R.rope_dynamic_ntk_theta(theta, D, f, L, L0)
    assert got == pytest.approx(oracle.dynamic_ntk_theta(theta, D, f, L, L0), rel=2 ** -23)
    if L <= L0:
        assert got == theta


@pytest.mark.parametrize("args", [(0.0, 128, 2.0), (1e4, 2, 2.0), (1e4, 127, 2.0), (1e4, 128, 0.0),
                                  (1e4, 128, float("nan")), (3e38, 128, 4.0)])
def test_ntk_theta_rejects(args):
    out = ctypes.c_float()
    assert R.lib().rope_ntk_theta(*args, ctypes.byref(out)) == BD.EINVAL
    assert R.lib().rope_ntk_theta(1e4, 128, 2.0, None) == BD.EINVAL


@pytest.mark.parametrize("args", [(1e4, 128, 0.0, 8192, 4096), (1e4, 128, 2.0, 0, 4096), (1e4, 128, 2.0, 10, 0),
                                  (1e4, 6, -1.0, 10, 4), (1e4, 3, 2.0, 10, 4)])
def test_dynamic_ntk_theta_rejects(args):
    out = ctypes.c_float()
    assert R.lib().rope_dynamic_ntk_theta(*args, ctypes.byref(out)) == BD.EINVAL


@pytest.mark.parametrize("args", [
    dict(mask=None), dict(mask_heads=2), dict(mask_ld=3), dict(out_is_mask=True), dict(Hq=6, Hkv=4),
    dict(causal=2), dict(scale=0.0), dict(D=7), dict(dt=4),
])
def test_prefill_masked_rejects(args):
    a = dict(mask=A[3], B=1, S=4, Hq=8, Hkv=2, D=64, mask_heads=1, mask_ld=4, causal=1, scale=0.125, dt=0)
    a.update(args)
    out = a["mask"] if args.get("out_is_mask") else A[4]
    st = R.lib().attn_prefill_masked(A[0], A[1], A[2], a["mask"], out, a["B"], a["S"], a["Hq"], a["Hkv"], a["D"],
                                     a["mask_heads"], a["mask_ld"], a["causal"], a["scale"], a["dt"], None)
    assert st == BD.EINVAL


def test_prefill_masked_unsupported_head_dim():
    assert R.lib().attn_prefill_masked(A[0], A[1], A[2], A[3], A[4], 1, 4, 8, 2, 96, 8, 4, 1, 0.1, 0, None) \
        == BD.EUNSUPPORTED
