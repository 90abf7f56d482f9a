"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws numbers and rounds them to the run dtype; it holds no
step of the method.  Every tensor is drawn from
``numpy.random.Generator(PCG64(seed))`` with ``standard_normal(dtype=float32)``
(N(0,1)), in the order listed per workload, and for bf16 runs rounded to
bfloat16 with round-to-nearest-even on the float32 bits.  Arrays are returned
as numpy: float32 for fp32 runs, uint16 bit patterns for bf16 runs; ``to_f64``
upcasts either exactly.

Workloads (LLaMA-shaped; seed = 1000 + workload number):

* ``c1``  tiny causal GQA prefill, fp32: B=1 S=128 Hq=8 Hkv=2 D=64, RoPE theta 1e4
* ``c2a`` unmasked MHA, bf16: B=4 S=128 Hq=Hkv=32 D=128 (hidden 4096), no RoPE
* ``c2b`` same shapes, causal with RoPE theta 1e4
* ``c3``  LLaMA-7B-shaped causal MHA prefill, bf16: B=2 S=4096 Hq=Hkv=32 D=128
* ``c4a`` LLaMA-70B-shaped causal GQA prefill, bf16: B=1 S=4096 Hq=64 Hkv=8 D=128
* ``c4b`` one GPU's 8-query-head / 1-KV-head share of c4a at the same S
* ``c5``  GQA decode, bf16: B=64 Hq=64 Hkv=8 D=128, context lengths uniform in
          [512, 8192], RoPE theta 1e4 with linear factor 2 at position = context
"""
import math
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Prefill:
    name: str
    B: int
    S: int
    Hq: int
    Hkv: int
    D: int
    causal: bool
    rope: bool
    dtype: str           # "bf16" | "fp32"
    seed: int
    theta: float = 10000.0
    factor: float = 1.0

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.D)

    def flops(self):
        """Algorithmic attention flops: 4*D per unmasked (query, key) pair per head."""
        pairs = self.S * (self.S + 1) // 2 if self.causal else self.S * self.S
        return 4.0 * self.D * pairs * self.B * self.Hq


@dataclass(frozen=True)
class Decode:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    ctx_lo: int
    ctx_hi: int
    dtype: str
    seed: int
    theta: float = 10000.0
    factor: float = 2.0

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.D)

    @property
    def max_kv(self):
        return self.ctx_hi + 1


WORKLOADS = {
    "c1": Prefill("tiny causal GQA prefill fp32", 1, 128, 8, 2, 64, True, True, "fp32", 1001),
    "c2a": Prefill("unmasked MHA bf16 S=128", 4, 128, 32, 32, 128, False, False, "bf16", 1002),
    "c2b": Prefill("causal MHA + RoPE bf16 S=128", 4, 128, 32, 32, 128, True, True, "bf16", 1002),
    "c3": Prefill("LLaMA-7B-shaped causal MHA prefill", 2, 4096, 32, 32, 128, True, True, "bf16", 1003),
    "c4a": Prefill("LLaMA-70B-shaped causal GQA prefill", 1, 4096, 64, 8, 128, True, True, "bf16", 1004),
    "c4b": Prefill("8q/1kv local head share of the 70B shape", 1, 4096, 8, 1, 128, True, True, "bf16", 1004),
    "c5": Decode("GQA decode against a bf16 KV cache", 64, 64, 8, 128, 512, 8192, "bf16", 1005),
}


def round_bf16(x32):
    """float32 array -> uint16 bfloat16 bit patterns, round to nearest even."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    u = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (u >> np.uint32(16)).astype(np.uint16)


def to_f64(a, dtype):
    """Exact upcast of a generated array (fp32, or uint16 bf16 bits) to float64."""
    if dtype == "bf16":
        return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def draw(rng, shape, dtype):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return round_bf16(x) if dtype == "bf16" else x


def prefill_inputs(w, seed=None):
    """q [B,S,Hq,D], k [B,S,Hkv,D], v [B,S,Hkv,D], drawn in that order."""
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    q = draw(rng, (w.B, w.S, w.Hq, w.D), w.dtype)
    k = draw(rng, (w.B, w.S, w.Hkv, w.D), w.dtype)
    v = draw(rng, (w.B, w.S, w.Hkv, w.D), w.dtype)
    return q, k, v


def decode_inputs(w, seed=None, B=None):
    """Decode inputs, drawn in this order:

    ctx [B] int in [ctx_lo, ctx_hi]; q [B,Hq,D]; k_new, v_new [B,Hkv,D];
    then per sequence b: k_cache[b], v_cache[b] ([Hkv, max_kv, D] each).
    The cache holds (already rotated) keys at rows 0..ctx-1; the new token
    goes to row ctx, so kv_len = ctx + 1.  ``B`` draws only the first B
    sequences of the same stream.
    """
    B = w.B if B is None else B
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    ctx = rng.integers(w.ctx_lo, w.ctx_hi + 1, size=w.B).astype(np.int32)[:B]
    q = draw(rng, (w.B, w.Hq, w.D), w.dtype)[:B]
    k_new = draw(rng, (w.B, w.Hkv, w.D), w.dtype)[:B]
    v_new = draw(rng, (w.B, w.Hkv, w.D), w.dtype)[:B]
    dt = np.uint16 if w.dtype == "bf16" else np.float32
    k_cache = np.empty((B, w.Hkv, w.max_kv, w.D), dtype=dt)
    v_cache = np.empty((B, w.Hkv, w.max_kv, w.D), dtype=dt)
    for b in range(B):
        k_cache[b] = draw(rng, (w.Hkv, w.max_kv, w.D), w.dtype)
        v_cache[b] = draw(rng, (w.Hkv, w.max_kv, w.D), w.dtype)
    return dict(ctx=ctx, q=q, k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache)


def random_case(seed, shape, dtype):
    """One N(0,1) tensor of any shape (edge-case tests)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return draw(rng, shape, dtype)
