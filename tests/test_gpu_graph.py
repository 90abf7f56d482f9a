"""The entry points under HIP graph capture: they allocate nothing and issue no
memsets, so a serving loop can capture them.  Each captured sequence is
replayed several times on fresh inputs copied into its static buffers, with
eager work and synchronisations in between, and every replay must equal the
same calls run eagerly, bit for bit."""
import numpy as np
import pytest

import rope_causal_gqa_amd as R
from rope_causal_gqa_amd import workloads as W
from tests.gpu_helpers import announce, dev

pytestmark = pytest.mark.gpu


def _i32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def test_graph_prefill_paths():
    """rope_apply + attn_prefill (8-wave grid), attn_prefill on a four-key-group
    grid, attn_prefill_ws (stream-K: per-tile counters that every call leaves
    at zero, so replays find them ready) and rope_attn_prefill, captured
    together."""
    import torch
    announce("graph: prefill paths")
    B, S, Hq, Hkv, D = 2, 2048, 32, 32, 128      # paired 8-wave grid
    q, k, v = (dev(W.random_case(s, (B, S, h, D), "bf16"), "bf16") for s, h in ((1, Hq), (2, Hkv), (3, Hkv)))
    q2, k2, v2 = (dev(W.random_case(s, (1, 2100, h, D), "bf16"), "bf16") for s, h in ((4, 8), (5, 1), (6, 1)))
    q3, k3, v3 = (dev(W.random_case(s, (1, 4096, h, D), "bf16"), "bf16") for s, h in ((8, 8), (9, 1), (10, 1)))
    out, out2, out3 = torch.empty_like(q), torch.empty_like(q2), torch.empty_like(q3)
    wsk = torch.zeros(R.attn_prefill_workspace_bytes(1, 4096, 8, D, True), dtype=torch.uint8, device="cuda")
    assert wsk.numel() > 0
    qf, kf = q.clone(), k.clone()
    outf = torch.empty_like(q)
    ws = torch.empty(R.rope_attn_prefill_workspace_bytes(B, S, D), dtype=torch.uint8, device="cuda")

    def calls():
        R.rope_apply(q, k, None, 1e4, 1.0)
        R.attn_prefill(q, k, v, out, causal=True, scale=D ** -0.5)
        R.attn_prefill(q2, k2, v2, out2, causal=True, scale=D ** -0.5)
        R.attn_prefill_ws(q3, k3, v3, out3, causal=True, scale=D ** -0.5, workspace=wsk)
        R.rope_attn_prefill(qf, kf, v, None, outf, causal=True, scale=D ** -0.5, theta=1e4, workspace=ws)

    srcs = [tuple(dev(W.random_case(100 * r + s, t.shape, "bf16"), "bf16")
                  for s, t in enumerate((q, k, v, q2, k2, v2, q3, k3, v3))) for r in range(3)]

    def load(r):
        for dst, src in zip((q, k, v, q2, k2, v2, q3, k3, v3), srcs[r]):
            dst.copy_(src)
        qf.copy_(srcs[r][0])
        kf.copy_(srcs[r][1])

    # eager references
    refs = []
    for r in range(3):
        load(r)
        calls()
        torch.cuda.synchronize()
        refs.append([t.clone() for t in (q, k, out, out2, out3, kf, outf)])
    # capture (after a warm-up on the side stream, as torch requires)
    load(0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    load(0)
    with torch.cuda.graph(g):
        calls()
    for rep in range(2):
        for r in range(3):
            load(r)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for got, ref in zip((q, k, out, out2, out3, kf, outf), refs[r]):
                assert torch.equal(got, ref), f"replay {rep}/{r} differs from the eager calls"


def test_graph_decode_paths():
    """rope_apply + kv_append + attn_decode and rope_attn_decode, captured."""
    import torch
    announce("graph: decode paths")
    w = W.WORKLOADS["c5"]
    B, Hq, Hkv, D, max_kv = 8, w.Hq, w.Hkv, w.D, 1500
    lens = _i32([1, 700, 1500, 1200, 3, 999, 1024, 64])
    pos = _i32(np.array([0, 699, 1499, 1199, 2, 998, 1023, 63]).reshape(B, 1))
    bufs = {n: dev(W.random_case(7 + i, shp, "bf16"), "bf16") for i, (n, shp) in enumerate(
        (("q", (B, 1, Hq, D)), ("kn", (B, 1, Hkv, D)), ("vn", (B, Hkv, D)),
         ("kc", (B, Hkv, max_kv, D)), ("vc", (B, Hkv, max_kv, D))))}
    kc2, vc2 = bufs["kc"].clone(), bufs["vc"].clone()
    q2, kn2 = bufs["q"].clone(), bufs["kn"].clone()
    out, out2 = (torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda") for _ in range(2))
    ws = torch.empty(R.attn_decode_workspace_bytes(B, Hq, D, max_kv), dtype=torch.uint8, device="cuda")
    ws2 = torch.empty(R.rope_attn_decode_workspace_bytes(B, Hq, D, max_kv), dtype=torch.uint8, device="cuda")

    def calls():
        R.rope_apply(bufs["q"], bufs["kn"], pos, w.theta, w.factor)
        R.kv_append(bufs["kc"], bufs["vc"], bufs["kn"].view(B, Hkv, D), bufs["vn"], _slots)
        R.attn_decode(bufs["q"].view(B, Hq, D), bufs["kc"], bufs["vc"], lens, out, scale=w.scale, workspace=ws)
        R.rope_attn_decode(q2.view(B, Hq, D), kn2.view(B, Hkv, D), bufs["vn"], kc2, vc2, lens, None, out2,
                           scale=w.scale, theta=w.theta, linear_factor=w.factor, workspace=ws2)

    _slots = _i32(np.array([0, 699, 1499, 1199, 2, 998, 1023, 63]))
    srcs = [{n: dev(W.random_case(1000 * (r + 1) + i, t.shape, "bf16"), "bf16") for i, (n, t) in enumerate(bufs.items())}
            for r in range(3)]

    def load(r):
        for n, t in bufs.items():
            t.copy_(srcs[r][n])
        kc2.copy_(srcs[r]["kc"])
        vc2.copy_(srcs[r]["vc"])
        q2.copy_(srcs[r]["q"])
        kn2.copy_(srcs[r]["kn"])

    watched = lambda: (out, out2, bufs["kc"], bufs["vc"], kc2, vc2)
    refs = []
    for r in range(3):
        load(r)
        calls()
        torch.cuda.synchronize()
        refs.append([t.clone() for t in watched()])
    load(0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    load(0)
    with torch.cuda.graph(g):
        calls()
    for rep in range(2):
        for r in range(3):
            load(r)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for got, ref in zip(watched(), refs[r]):
                assert torch.equal(got, ref), f"replay {rep}/{r} differs from the eager calls"
