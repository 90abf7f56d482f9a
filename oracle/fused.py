"""Rotation followed by attention, float64 oracle (test infrastructure only).

Definition followed: the forward order of "【HuggingFace Transformers】
LlamaAttention源码解析", section 2 -- step 3 rotates the projected queries and
keys with the cos/sin of ``position_ids`` (and ``past_key_value.update`` keeps
the rotated keys), steps 4-5 run the attention on the rotated tensors.  For a
decode step, the new token's key and value are appended to the cache and its
query attends to every cached position and itself ("LLaMA2大语言模型架构详解",
section "KV cache"); the token's position is its index in the sequence.

Both functions are the plain composition of the oracle's own ``rope`` and
``attention`` functions, with nothing reordered or fused.
"""
import numpy as np

from .attention import attention, decode, kv_append
from .rope import rope_apply, rotate


def rope_attention(q, k, v, position_ids, causal, scale, theta, linear_factor=1.0):
    """Prefill: attention(rope(q), rope(k), v) for q [B,S,Hq,D], k/v [B,S,Hkv,D].

    ``position_ids`` [B,S] (None: 0..S-1).  Returns (out [B,S,Hq,D], rotated k),
    both float64.
    """
    q_rot, k_rot = rope_apply(q, k, position_ids, theta, linear_factor)
    return attention(q_rot, k_rot, np.asarray(v, dtype=np.float64), causal, scale), k_rot


def rope_decode_step(q, k_new, v_new, k_cache, v_cache, kv_lens, position_ids, scale, theta, linear_factor=1.0):
    """One decode step per sequence.

    q [B,Hq,D], k_new/v_new [B,Hkv,D], caches [B,Hkv,max_kv,D]; ``kv_lens[b]``
    counts the cached rows including the new token, whose row is
    ``kv_lens[b] - 1`` and whose position is ``position_ids[b]`` (None: that
    row index).  The new key is rotated at that position and stored with v_new
    (rows outside the cache are not written), the query is rotated at the same
    position and attends over the first kv_lens[b] rows.
    Returns (out [B,Hq,D], k_cache', v_cache'), float64.
    """
    kv_lens = np.asarray(kv_lens)
    slots = kv_lens - 1
    pos = slots if position_ids is None else np.asarray(position_ids)
    q_rot = rotate(q, pos[:, None], theta, linear_factor)
    k_rot = rotate(k_new, pos[:, None], theta, linear_factor)
    kc, vc = kv_append(k_cache, v_cache, k_rot, np.asarray(v_new, dtype=np.float64), slots)
    return decode(q_rot, kc, vc, kv_lens, scale), kc, vc
