"""Plain float64 CPU oracle for RoPE + causal grouped-query attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the tests, the smoke check and the CPU
baseline leg of the benchmark use it.  It shares no code with the HIP library
(no kernels, headers, tables or helpers) and imports nothing from it.

Every function materialises what the pages define, in numpy float64, with no
blocking, fusion or reordering beyond that definition:

* ``rope``      -- rotary position embedding (frequencies, angles, rotation).
* ``attention`` -- scaled dot-product attention with a bottom-right causal
                   mask (optionally a sliding window) and grouped-query head
                   sharing; single-token decode and chunked / variable-length
                   prefill against a cache.
* ``fused``     -- rotation then attention, as one prefill or one decode step
                   (with the cache append), composed from the two above.
* ``ntk``       -- NTK-aware scaling of the RoPE base (static and dynamic).

Pins (tests marked ``not gpu``) tie each function to something other than
itself: closed forms, invariants, brute-force loops on tiny shapes, a library
routine the pages name (torch's CPU scaled_dot_product_attention in float64),
and hand-derived fixtures under ``tests/golden``.
"""
from .rope import inv_freq, angles, rotate, rope_apply
from .attention import attention, attention_cache, attention_probs, decode, kv_append
from .fused import rope_attention, rope_decode_step
from .ntk import ntk_theta, dynamic_ntk_theta

__all__ = ["inv_freq", "angles", "rotate", "rope_apply",
           "attention", "attention_cache", "attention_probs", "decode", "kv_append",
           "rope_attention", "rope_decode_step", "ntk_theta", "dynamic_ntk_theta"]
