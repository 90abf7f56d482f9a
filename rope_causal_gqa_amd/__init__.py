"""rope_causal_gqa_amd: RoPE + causal grouped-query attention on MI355X (gfx950).

The compute lives in ``librcgqa.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/rcgqa.h``).  This package is a thin ctypes binding over
it: it reads shapes and device pointers off torch tensors and passes them on;
it never computes any step itself.  The library is loaded on first use and a
missing or unloadable library raises immediately.
"""
from ._binding import (RcgqaError, attn_decode, attn_decode_noalloc, attn_decode_workspace_bytes, attn_prefill,
                       attn_prefill_cache, attn_prefill_cache_workspace_bytes, attn_prefill_cache_ws,
                       attn_prefill_masked, attn_prefill_workspace_bytes, attn_prefill_ws, kv_append, lib, lib_path, rope_apply, rope_apply_interleaved,
                       rope_attn_decode, rope_attn_decode_workspace_bytes, rope_attn_prefill,
                       rope_attn_prefill_workspace_bytes, rope_dynamic_ntk_theta, rope_ntk_theta)

__all__ = ["RcgqaError", "attn_decode", "attn_decode_noalloc", "attn_decode_workspace_bytes", "attn_prefill",
           "attn_prefill_cache", "attn_prefill_cache_workspace_bytes", "attn_prefill_cache_ws",
           "attn_prefill_masked", "attn_prefill_workspace_bytes", "attn_prefill_ws", "kv_append", "lib", "lib_path", "rope_apply", "rope_apply_interleaved",
           "rope_attn_decode", "rope_attn_decode_workspace_bytes", "rope_attn_prefill",
           "rope_attn_prefill_workspace_bytes", "rope_dynamic_ntk_theta", "rope_ntk_theta"]
