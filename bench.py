"""Benchmark of the RoPE + causal GQA hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  prefill  (LLaMA-7B-shaped, B=2 S=4096 Hq=Hkv=32 D=128 bf16):
           rope_apply on Q/K in place, then causal attn_prefill;
  decode   (B=64 Hq=64 Hkv=8 D=128 bf16, context lengths uniform in [512, 8192]):
           rope_apply on q / k_new at position = context (linear factor 2),
           kv_append at row = context, attn_decode over context + 1 rows.
Decode alternates between two separately allocated caches so consecutive
steps never find the previous step's cache in the 256 MB Infinity Cache.

Prints ONE JSON line.  `value` is the prefill attention throughput in TFLOP/s
(algorithmic flops: 4*D per unmasked query-key pair per head, over the
attn_prefill launch time measured with HIP events on the launch stream); the
decode figure (GB/s of K/V bytes read, each row once per GQA group) rides in
`decode`.  `roofline` is for the prefill kernel against the bf16 dense MFMA
peak; `decode.roofline` against HBM.  `chunked_prefill` and `sliding_window`
time the two prefill extensions (attn_prefill_cache) separately, after the
timed steps; `gqa_prefill` times attn_prefill on the LLaMA-70B-shaped GQA
prefill (B=1 S=4096 Hq=64 Hkv=8 D=128) and, on its 8-query-head / 1-KV-head
share, the stream-K entry point attn_prefill_ws (attn_prefill alongside);
`stream_k_prefill` times attn_prefill_ws against attn_prefill on four more causal
shapes that the launcher runs on unpaired grids, and attn_prefill_cache_ws against
attn_prefill_cache on two chunked prefills; `fused_rope_prefill` / `fused_rope_decode` time the fused RoPE
entry points against the separate calls on the same workloads; `ntk_rope`
times rope_apply at an NTK-aware scaled base; `masked_prefill` times
attn_prefill_masked (causal plus a key-padding mask) on LLaMA-7B-shaped heads;
`small_configs` times RoPE and attention on the three small workloads (tiny fp32
GQA, S=128 MHA unmasked and causal with RoPE).  `cpu_baseline` times the float64
oracle on a bounded sample on the host cores.

Before the W warm-up steps the step runs untimed for --settle-s seconds
(default 2): under sustained MFMA load the GPU lowers its clock within the
first second or so, and a short run would otherwise be timed on that ramp.
The settle time and step count are reported in `settle`.

    python bench.py [--steps K] [--warmup W] [--settle-s S] [--gpus 1] [--no-cpu-baseline] [--no-extras]
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill attention TFLOP/s (% MFMA peak) + decode KV-cache GB/s (% HBM peak)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
PREFILL_KERNEL_SRC = os.path.join(ROOT, "rope_causal_gqa_amd", "csrc", "prefill_bf16.hip")
DECODE_KERNEL_SRC = os.path.join(ROOT, "rope_causal_gqa_amd", "csrc", "decode.hip")


def _sha(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def _traffic(name, src):
    """HBM bytes per launch from committed rocprofv3 --pmc summaries, only if they
    were taken on the current kernel source."""
    p = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("kernel_src_sha") != _sha(src):
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(budget_s=12.0):
    """Time the float64 oracle on a bounded sample of the prefill workload:
    whole (batch, head) rows of the causal S=4096 attention, RoPE included."""
    import oracle
    from rope_causal_gqa_amd import workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    w = W.WORKLOADS["c3"]
    rng = np.random.Generator(np.random.PCG64(w.seed))
    done, flops = 0, 0.0
    t0 = time.perf_counter()
    while done == 0 or time.perf_counter() - t0 < budget_s:
        q = W.to_f64(W.draw(rng, (1, w.S, 1, w.D), "bf16"), "bf16")
        k = W.to_f64(W.draw(rng, (1, w.S, 1, w.D), "bf16"), "bf16")
        v = W.to_f64(W.draw(rng, (1, w.S, 1, w.D), "bf16"), "bf16")
        qr, kr = oracle.rope_apply(q, k, None, w.theta, w.factor)
        oracle.attention(qr, kr, v, True, w.scale)
        done += 1
        flops += 4.0 * w.D * (w.S * (w.S + 1) // 2)
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} whole (batch, head) pairs of the B=2 S=4096 D=128 causal prefill "
                      f"(RoPE + attention, float64 numpy) in {dt:.1f} s; cpus visible "
                      f"{len(os.sched_getaffinity(0))}"}


def cpu_oracle_configs():
    """Seconds of the float64 oracle on the small workloads (C1, C2a, C2b: whole,
    RoPE included where the workload has it) and on the first 8 sequences of the
    decode workload (rotation, append and decode), for the baseline table."""
    import oracle
    from rope_causal_gqa_amd import workloads as W
    out = {}
    for name in ("c1", "c2a", "c2b"):
        w = W.WORKLOADS[name]
        q, k, v = (W.to_f64(a, w.dtype) for a in W.prefill_inputs(w))
        t0 = time.perf_counter()
        if w.rope:
            q, k = oracle.rope_apply(q, k, None, w.theta, w.factor)
        oracle.attention(q, k, v, w.causal, w.scale)
        out[name] = {"seconds": round(time.perf_counter() - t0, 4), "sample": "whole workload"}
    w = W.WORKLOADS["c5"]
    nb = 8
    inp = W.decode_inputs(w, B=nb)
    f = lambda a: W.to_f64(a, w.dtype)
    t0 = time.perf_counter()
    ctx = inp["ctx"]
    oracle.rope_decode_step(f(inp["q"]), f(inp["k_new"]), f(inp["v_new"]), f(inp["k_cache"]), f(inp["v_cache"]),
                            ctx + 1, None, w.scale, w.theta, w.factor)
    dt = time.perf_counter() - t0
    kv_bytes = float(np.sum(ctx.astype(np.int64) + 1)) * w.Hkv * w.D * 2 * 2
    out["c5"] = {"seconds": round(dt, 4), "sample": f"first {nb} of {w.B} sequences",
                 "gbps": round(kv_bytes / dt / 1e9, 3)}
    return out


def _time_launches(fn, stream, warmup=20, reps=200):
    """Mean time (ms) of one launch of fn, HIP events on the launch stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def _next_rows(R, dev, stream):
    """Throughput of the two prefill extensions on LLaMA-7B-shaped heads
    (Hq = Hkv = 32, D = 128, bf16, causal), outside the timed step:
    * chunked prefill: B=2, a chunk of 512 new tokens at the end of a
      4608-token cache (kv_lens = 4608);
    * sliding window: B=2, S=4096 prefill through the cache entry point with
      window 1024.
    Algorithmic flops = 4*D per visible (query, key) pair per head."""
    import torch
    D, H, B = 128, 32, 2
    g = torch.Generator(device=dev)
    g.manual_seed(2024)
    out = {}
    for name, Sq, L, window in (("chunked_prefill", 512, 4608, 0), ("sliding_window", 4096, 4096, 1024)):
        q = torch.randn((B, Sq, H, D), generator=g, device=dev).to(torch.bfloat16)
        kc = torch.randn((B, H, L, D), generator=g, device=dev).to(torch.bfloat16)
        vc = torch.randn((B, H, L, D), generator=g, device=dev).to(torch.bfloat16)
        lens = torch.full((B,), L, dtype=torch.int32, device=dev)
        o = torch.empty_like(q)
        pos = np.arange(Sq, dtype=np.int64) + (L - Sq)
        seen = np.minimum(pos + 1, window) if window else pos + 1
        flops = 4.0 * D * H * B * float(seen.sum())
        ms = _time_launches(lambda: R.attn_prefill_cache(q, kc, vc, lens, o, causal=True, scale=D ** -0.5,
                                                         window=window), stream)
        tf = flops / (ms * 1e-3) / 1e12
        out[name] = {"workload": f"B={B} Hq=Hkv={H} D={D} bf16 causal, Sq={Sq} new tokens, kv_len={L}"
                                 + (f", window={window}" if window else ""),
                     "value": round(tf, 2), "unit": "TFLOP/s", "launch_ms": round(ms, 4),
                     "algorithmic_flops": flops,
                     "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                                  "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4)}}
        del q, kc, vc, o
    # general additive mask: key padding (sequence 1 keeps 3000 of its 4096 keys) on top of the causal mask
    Sm, lens_m = 4096, (4096, 3000)
    q = torch.randn((B, Sm, H, D), generator=g, device=dev).to(torch.bfloat16)
    k = torch.randn((B, Sm, H, D), generator=g, device=dev).to(torch.bfloat16)
    v = torch.randn((B, Sm, H, D), generator=g, device=dev).to(torch.bfloat16)
    mask = torch.zeros((B, 1, Sm, Sm), dtype=torch.bfloat16, device=dev)
    for b, L in enumerate(lens_m):
        mask[b, :, :, L:] = float("-inf")
    o = torch.empty_like(q)
    ms = _time_launches(lambda: R.attn_prefill_masked(q, k, v, mask, o, causal=True, scale=D ** -0.5), stream)
    i = np.arange(Sm)
    flops = 4.0 * D * H * float(sum(np.minimum(i + 1, L).sum() for L in lens_m))
    tf = flops / (ms * 1e-3) / 1e12
    out["masked_prefill"] = {"workload": f"B={B} S={Sm} Hq=Hkv={H} D={D} bf16 causal + key-padding mask "
                                         f"[B,1,S,S] (keys kept {lens_m})",
                             "value": round(tf, 2), "unit": "TFLOP/s", "launch_ms": round(ms, 4),
                             "algorithmic_flops": flops,
                             "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                                          "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4)}}
    del q, k, v, o, mask
    from rope_causal_gqa_amd import workloads as W
    gqa = {}
    for name in ("c4a", "c4b"):
        w = W.WORKLOADS[name]
        q = torch.randn((w.B, w.S, w.Hq, w.D), generator=g, device=dev).to(torch.bfloat16)
        k = torch.randn((w.B, w.S, w.Hkv, w.D), generator=g, device=dev).to(torch.bfloat16)
        v = torch.randn((w.B, w.S, w.Hkv, w.D), generator=g, device=dev).to(torch.bfloat16)
        o = torch.empty_like(q)
        ms = _time_launches(lambda: R.attn_prefill(q, k, v, o, causal=True, scale=w.scale), stream)
        entry = "attn_prefill"
        need = R.attn_prefill_workspace_bytes(w.B, w.S, w.Hq, w.D, True)
        plain_ms = ms
        if need:
            # small grids: the stream-K entry point (workspace zeroed once, reused)
            wsp = torch.zeros(need, dtype=torch.uint8, device=dev)
            ms = _time_launches(lambda: R.attn_prefill_ws(q, k, v, o, causal=True, scale=w.scale, workspace=wsp),
                                stream)
            entry = "attn_prefill_ws"
            del wsp
        tf = w.flops() / (ms * 1e-3) / 1e12
        gqa[name] = {"workload": f"{w.name}: B={w.B} S={w.S} Hq={w.Hq} Hkv={w.Hkv} D={w.D} bf16 causal",
                     "entry": entry, "value": round(tf, 2), "unit": "TFLOP/s", "launch_ms": round(ms, 4),
                     "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                                  "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4)}}
        if need:
            gqa[name]["attn_prefill_launch_ms"] = round(plain_ms, 4)
            gqa[name]["attn_prefill_tflops"] = round(w.flops() / (plain_ms * 1e-3) / 1e12, 2)
        del q, k, v, o
    out["gqa_prefill"] = [gqa["c4a"], gqa["c4b"]]
    # attn_prefill_ws against attn_prefill on causal shapes the launcher runs on
    # unpaired grids (one GPU's share of a head split, long single sequences)
    rows = []
    for B, S, Hq, Hkv in ((1, 4096, 16, 2), (1, 8192, 8, 1), (1, 16384, 4, 1), (4, 2048, 8, 1)):
        D = 128
        q = torch.randn((B, S, Hq, D), generator=g, device=dev).to(torch.bfloat16)
        k = torch.randn((B, S, Hkv, D), generator=g, device=dev).to(torch.bfloat16)
        v = torch.randn((B, S, Hkv, D), generator=g, device=dev).to(torch.bfloat16)
        o = torch.empty_like(q)
        wsp = torch.zeros(max(R.attn_prefill_workspace_bytes(B, S, Hq, D, True), 1), dtype=torch.uint8, device=dev)
        ws_ms = _time_launches(lambda: R.attn_prefill_ws(q, k, v, o, causal=True, scale=D ** -0.5, workspace=wsp),
                               stream)
        ms = _time_launches(lambda: R.attn_prefill(q, k, v, o, causal=True, scale=D ** -0.5), stream)
        flops = 4.0 * D * Hq * B * (S * (S + 1) / 2)
        rows.append({"workload": f"B={B} S={S} Hq={Hq} Hkv={Hkv} D={D} bf16 causal",
                     "attn_prefill_ws_ms": round(ws_ms, 4), "attn_prefill_ms": round(ms, 4),
                     "attn_prefill_ws_tflops": round(flops / (ws_ms * 1e-3) / 1e12, 2),
                     "attn_prefill_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                     "speedup": round(ms / ws_ms, 3)})
        del q, k, v, o, wsp
    # and attn_prefill_cache_ws against attn_prefill_cache on chunks whose key-group grid underfills the GPU
    for B, Sq, Hq, Hkv, L in ((1, 2048, 8, 1, 8192), (2, 512, 16, 2, 16384)):
        D = 128
        q = torch.randn((B, Sq, Hq, D), generator=g, device=dev).to(torch.bfloat16)
        kc = torch.randn((B, Hkv, L, D), generator=g, device=dev).to(torch.bfloat16)
        vc = torch.randn((B, Hkv, L, D), generator=g, device=dev).to(torch.bfloat16)
        lens = torch.full((B,), L, dtype=torch.int32, device=dev)
        o = torch.empty_like(q)
        wsp = torch.zeros(max(R.attn_prefill_cache_workspace_bytes(B, Sq, Hq, D, L, True, 0), 1), dtype=torch.uint8,
                          device=dev)
        ws_ms = _time_launches(lambda: R.attn_prefill_cache_ws(q, kc, vc, lens, o, causal=True, scale=D ** -0.5,
                                                               workspace=wsp), stream)
        ms = _time_launches(lambda: R.attn_prefill_cache(q, kc, vc, lens, o, causal=True, scale=D ** -0.5), stream)
        flops = 4.0 * D * Hq * B * sum(L - Sq + i + 1 for i in range(Sq))
        rows.append({"workload": f"B={B} Sq={Sq} new tokens after {L - Sq} cached, Hq={Hq} Hkv={Hkv} D={D} bf16 causal",
                     "attn_prefill_cache_ws_ms": round(ws_ms, 4), "attn_prefill_cache_ms": round(ms, 4),
                     "attn_prefill_cache_ws_tflops": round(flops / (ws_ms * 1e-3) / 1e12, 2),
                     "attn_prefill_cache_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                     "speedup": round(ms / ws_ms, 3)})
        del q, kc, vc, o, wsp
    out["stream_k_prefill"] = rows
    return out


def _small_rows(R, dev, stream):
    """The three small workloads (tiny fp32 GQA prefill; S=128 MHA bf16 unmasked, and
    causal with RoPE), outside the timed step: RoPE and attention timed as separate
    launches on the seeded inputs (RoPE rotates them in place again on every launch,
    which does not change its cost).  Parity configurations, not bench lines: at
    these sizes a launch is bound by latency, not by the MFMA or HBM rooflines."""
    import torch
    from rope_causal_gqa_amd import workloads as W
    rows = []
    for name in ("c1", "c2a", "c2b"):
        w = W.WORKLOADS[name]
        if w.dtype == "fp32":
            q, k, v = (torch.from_numpy(np.ascontiguousarray(a)).to(dev) for a in W.prefill_inputs(w))
        else:
            q, k, v = (torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
                       for a in W.prefill_inputs(w))
        o = torch.empty_like(q)
        rope_ms = _time_launches(lambda: R.rope_apply(q, k, None, w.theta, w.factor), stream) if w.rope else 0.0
        attn_ms = _time_launches(lambda: R.attn_prefill(q, k, v, o, causal=w.causal, scale=w.scale), stream)
        rows.append({"workload": f"{name}: {w.name}, B={w.B} S={w.S} Hq={w.Hq} Hkv={w.Hkv} D={w.D}",
                     "dtype": w.dtype, "rope_us": round(rope_ms * 1e3, 1), "attention_us": round(attn_ms * 1e3, 1),
                     "attention_tflops": round(w.flops() / (attn_ms * 1e-3) / 1e12, 2)})
    return rows


def _fused_rows(R, wp, wd, q, k, v, out, dq, dkn, dvn, kc, vc, ctx_d, lens_d, pos_d, dout, ws, stream):
    """The fused RoPE paths against the separate calls, on the same two workloads
    (outside the timed step):
    * rope_attn_prefill (keys rotated in one pass that also writes the cos/sin
      rows, queries rotated as the attention kernel loads them) vs rope_apply on
      Q and K + attn_prefill;
    * rope_attn_decode (q / new-key rotation and cache append in one kernel,
      then the decode kernels) vs rope_apply + kv_append + attn_decode."""
    import torch
    dev = q.device
    pws = torch.empty(R.rope_attn_prefill_workspace_bytes(wp.B, wp.S, wp.D), dtype=torch.uint8, device=dev)
    dws = torch.empty(R.rope_attn_decode_workspace_bytes(wd.B, wd.Hq, wd.D, wd.max_kv), dtype=torch.uint8,
                      device=dev)
    fused_ms = _time_launches(lambda: R.rope_attn_prefill(q, k, v, None, out, causal=True, scale=wp.scale,
                                                          theta=wp.theta, workspace=pws), stream)

    def sep():
        R.rope_apply(q, k, None, wp.theta, wp.factor)
        R.attn_prefill(q, k, v, out, causal=True, scale=wp.scale)
    sep_ms = _time_launches(sep, stream)
    flops = wp.flops()
    dq3 = dq.view(wd.B, wd.Hq, wd.D)
    dkn3 = dkn.view(wd.B, wd.Hkv, wd.D)
    dfused_ms = _time_launches(lambda: R.rope_attn_decode(dq3, dkn3, dvn, kc, vc, lens_d, None, dout, scale=wd.scale,
                                                          theta=wd.theta, linear_factor=wd.factor, workspace=dws),
                               stream)

    def dsep():
        R.rope_apply(dq, dkn, pos_d, wd.theta, wd.factor)
        R.kv_append(kc, vc, dkn3, dvn, ctx_d)
        R.attn_decode(dq3, kc, vc, lens_d, dout, scale=wd.scale, workspace=ws)
    dsep_ms = _time_launches(dsep, stream)
    # NTK-aware scaling only changes the base handed to the RoPE kernel
    ntk_theta = R.rope_ntk_theta(wp.theta, wp.D, 8.0)
    ntk_ms = _time_launches(lambda: R.rope_apply(q, k, None, ntk_theta, 1.0), stream)
    rope_bytes = 2.0 * wp.B * wp.S * (wp.Hq + wp.Hkv) * wp.D * 2
    return {
        "ntk_rope": {
            "workload": f"rope_apply on the B=2 S=4096 Hq=Hkv=32 D=128 bf16 Q/K at the NTK-aware base for scale 8 "
                        f"(theta {ntk_theta:.1f})",
            "value": round(rope_bytes / (ntk_ms * 1e-3) / 1e9, 1), "unit": "GB/s", "launch_ms": round(ntk_ms, 4)},
        "fused_rope_prefill": {
            "workload": "B=2 S=4096 Hq=Hkv=32 D=128 bf16 causal, RoPE theta 1e4 + attention",
            "fused_ms": round(fused_ms, 4), "separate_ms": round(sep_ms, 4),
            "speedup": round(sep_ms / fused_ms, 3),
            "value": round(flops / (fused_ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s (attention flops / whole call)"},
        "fused_rope_decode": {
            "workload": "B=64 Hq=64 Hkv=8 D=128 bf16, RoPE factor 2 at position = context, append + decode",
            "fused_ms": round(dfused_ms, 4), "separate_ms": round(dsep_ms, 4),
            "speedup": round(dsep_ms / dfused_ms, 3)},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--settle-s", type=float, default=2.0,
                    help="seconds of untimed steps before the W warm-up steps, so the timed steps run at the "
                         "clock the GPU holds under this load rather than on its ramp")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the prefill-extension and fused-RoPE timings after the steps "
                         "(profiling runs that should see only the step's kernels)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(this library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import torch
    import rope_causal_gqa_amd as R
    from rope_causal_gqa_amd import workloads as W

    R.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # Reference point for HBM: a plain 1 GiB device-to-device copy (also the
    # calibration kernel for the FETCH_SIZE / WRITE_SIZE counters).
    ca = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    cb = torch.empty_like(ca)
    cb.copy_(ca)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(3):
        cb.copy_(ca)
    c1.record()
    torch.cuda.synchronize()
    copy_gbps = 3 * 2 * ca.numel() * 4 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del ca, cb

    # ---- prefill inputs (LLaMA-7B-shaped)
    wp = W.WORKLOADS["c3"]
    tb = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v = (tb(a) for a in W.prefill_inputs(wp))
    out = torch.empty_like(q)

    # ---- decode inputs (GQA decode, bf16 cache); the caches are drawn on the device
    wd = W.WORKLOADS["c5"]
    rng = np.random.Generator(np.random.PCG64(wd.seed))
    ctx = rng.integers(wd.ctx_lo, wd.ctx_hi + 1, size=wd.B).astype(np.int32)
    ctx_d = torch.from_numpy(ctx).to(dev)
    lens_d = ctx_d + 1
    pos_d = ctx_d.view(wd.B, 1).contiguous()
    gen = torch.Generator(device=dev)
    gen.manual_seed(wd.seed)
    dq = torch.randn((wd.B, 1, wd.Hq, wd.D), generator=gen, device=dev).to(torch.bfloat16)
    dkn = torch.randn((wd.B, 1, wd.Hkv, wd.D), generator=gen, device=dev).to(torch.bfloat16)
    dvn = torch.randn((wd.B, wd.Hkv, wd.D), generator=gen, device=dev).to(torch.bfloat16)
    caches = []
    for _ in range(2):
        kc = torch.empty((wd.B, wd.Hkv, wd.max_kv, wd.D), dtype=torch.bfloat16, device=dev)
        vc = torch.empty_like(kc)
        for b in range(wd.B):
            kc[b].copy_(torch.randn((wd.Hkv, wd.max_kv, wd.D), generator=gen, device=dev))
            vc[b].copy_(torch.randn((wd.Hkv, wd.max_kv, wd.D), generator=gen, device=dev))
        caches.append((kc, vc))
    dout = torch.empty((wd.B, wd.Hq, wd.D), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(R.attn_decode_workspace_bytes(wd.B, wd.Hq, wd.D, wd.max_kv), dtype=torch.uint8, device=dev)

    kv_bytes = float(np.sum(ctx.astype(np.int64) + 1)) * wd.Hkv * wd.D * 2 * 2
    dec_bytes = kv_bytes + 2 * wd.B * wd.Hq * wd.D * 2          # + q read + out write
    pre_flops = wp.flops()

    stream = torch.cuda.current_stream(dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)

    # Odd steps rotate by the negated positions, undoing the even step's
    # rotation (up to bf16 rounding), so the timed Q/K stay the seeded draw
    # rotated at most once instead of drifting over hundreds of rotations.
    neg_pos = -torch.arange(wp.S, dtype=torch.int32, device=dev).repeat(wp.B, 1).contiguous()

    def step(i, rec=None):
        kc, vc = caches[i % 2]
        if rec: rec[0].record(stream)
        R.rope_apply(q, k, None if i % 2 == 0 else neg_pos, wp.theta, wp.factor)
        if rec: rec[1].record(stream)
        R.attn_prefill(q, k, v, out, causal=True, scale=wp.scale)
        if rec: rec[2].record(stream)
        R.rope_apply(dq, dkn, pos_d, wd.theta, wd.factor)
        R.kv_append(kc, vc, dkn.view(wd.B, wd.Hkv, wd.D), dvn, ctx_d)
        if rec: rec[3].record(stream)
        R.attn_decode(dq.view(wd.B, wd.Hq, wd.D), kc, vc, lens_d, dout, scale=wd.scale, workspace=ws)
        if rec: rec[4].record(stream)

    settle_steps, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < args.settle_s:
        for _ in range(10):
            step(settle_steps)
            settle_steps += 1
        torch.cuda.synchronize()
    settle_s = time.perf_counter() - t0
    for i in range(args.warmup):
        step(settle_steps + i)
    torch.cuda.synchronize()
    recs = [[ev() for _ in range(5)] for _ in range(args.steps)]
    t_start, t_end = ev(), ev()
    torch.cuda.synchronize()
    t_start.record(stream)
    first = settle_steps + args.warmup  # keeps the +/- rotation alternation
    for i in range(args.steps):
        step(first + i, recs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    rope_ms = np.array([r[0].elapsed_time(r[1]) for r in recs])
    pre_ms = np.array([r[1].elapsed_time(r[2]) for r in recs])
    dec_ms = np.array([r[3].elapsed_time(r[4]) for r in recs])

    pre_tflops = pre_flops / (pre_ms.mean() * 1e-3) / 1e12
    dec_gbps = dec_bytes / (dec_ms.mean() * 1e-3) / 1e9
    rope_bytes = 2.0 * wp.B * wp.S * (wp.Hq + wp.Hkv) * wp.D * 2
    extras, fused, small = {}, {}, None
    if not args.no_extras:
        extras = _next_rows(R, dev, stream)
        small = _small_rows(R, dev, stream)
        fused = _fused_rows(R, wp, wd, q, k, v, out, dq, dkn, dvn, caches[0][0], caches[0][1], ctx_d, lens_d,
                            pos_d, dout, ws, stream)
    res = {
        "metric": METRIC,
        "value": round(pre_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"seconds": round(settle_s, 2), "steps": settle_steps},
        "ms_per_step": round(total_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "LLaMA-7B-shaped causal MHA prefill B=2 S=4096 Hq=Hkv=32 D=128 + "
                               "GQA decode B=64 Hq=64 Hkv=8 D=128 ctx~U[512,8192]",
                   "global_batch": wp.B, "seq_len": wp.S, "parallelism": "single-gpu"},
        "roofline": {"bound": "mfma", "achieved": round(pre_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(pre_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": _traffic("prefill_c3", PREFILL_KERNEL_SRC),
                     "kernel": "prefill_bf16_kernel<128, 8, false, 1, 64, false, false>", "launch_ms": round(float(pre_ms.mean()), 4)},
        "decode": {"metric": "decode KV-cache GB/s", "value": round(dec_gbps, 1), "unit": "GB/s",
                   "launch_ms": round(float(dec_ms.mean()), 4),
                   "algorithmic_bytes": dec_bytes,
                   "roofline": {"bound": "hbm", "achieved": round(dec_gbps, 1), "peak": PEAK_HBM_GBPS,
                                "unit": "GB/s", "frac": round(dec_gbps / PEAK_HBM_GBPS, 4),
                                "traffic": _traffic("decode_c5", DECODE_KERNEL_SRC)}},
        "rope": {"value": round(rope_bytes / (rope_ms.mean() * 1e-3) / 1e9, 1), "unit": "GB/s",
                 "launch_ms": round(float(rope_ms.mean()), 4)},
        "hbm_copy_gbps": round(copy_gbps, 1),
        "chunked_prefill": extras.get("chunked_prefill"),
        "sliding_window": extras.get("sliding_window"),
        "gqa_prefill": extras.get("gqa_prefill"),
        "stream_k_prefill": extras.get("stream_k_prefill"),
        "masked_prefill": extras.get("masked_prefill"),
        "fused_rope_prefill": fused.get("fused_rope_prefill"),
        "fused_rope_decode": fused.get("fused_rope_decode"),
        "ntk_rope": fused.get("ntk_rope"),
        "small_configs": small,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline()
        res["cpu_oracle_configs"] = cpu_oracle_configs()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
