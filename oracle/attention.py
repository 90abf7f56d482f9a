"""Scaled dot-product attention, float64 oracle (test infrastructure only).

Definition followed ("【HuggingFace Transformers】LlamaAttention源码解析",
section 1.2 steps 2-4 and section 2 forward steps 4-5):

* scores = scale * Q K^T per head, with scale = 1/sqrt(d_k) by default and
  passed in by the caller (the ``scaling`` argument of the verl page, section
  "4.48+ 版本的主要区别");
* an additive mask (section 1.2 step 3: the mask is sliced to the query and
  key lengths and added to the scaled scores): the causal one, with -inf on
  masked entries so they get exactly zero weight, and optionally a general
  one given as an array [B, Hm, Sq, Sk] (Hm = 1: shared by all query heads,
  Hm = Hq: one per head) added to the scaled scores as it is.  Alignment (a reading): query i of Sq sits at
  absolute position Sk - Sq + i, so it sees keys j <= i + (Sk - Sq); with
  Sq == Sk this is the usual lower triangle;
* softmax over keys, then weights @ V;
* grouped-query sharing: query head h reads K/V head h // G with
  G = Hq / Hkv, the index map of ``repeat_kv`` in section 2 step 4, and of
  "8 query heads share one K/V head" ("Llama2 Transformer架构解析与优化实践",
  section 2.1);
* decode with a cache ("LLaMA2大语言模型架构详解", section "KV cache"): one new
  query against all kv_len cached (already rotated) keys and values;
* chunked / variable-length prefill against a cache: a block of Sq new queries
  of sequence b against its kv_len_b cached rows, the last Sq of which are the
  block's own keys (the bottom-right alignment above with Sk = kv_len_b; the
  variable-length support of "【HuggingFace Transformers】LlamaAttention源码解析",
  section 3.1);
* sliding window: the flash-attention call of "llama.py — LLaMA 注意力层 Ulysses
  SP 适配" (section "第二步：RoPE + Flash Attention") passes a ``sliding_window``,
  never defined on the pages.  Reading: with window W > 0 a query at absolute
  position p sees only the W most recent positions, keys p - W < j <= p (causal
  only); W = 0 means no window.

A row whose keys are all masked (possible only when Sq > Sk, or kv_len == 0)
returns zeros (a reading: the pages never produce such a row).
"""
import numpy as np


def _check(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, S, H, D]")
    B, Sq, Hq, D = q.shape
    if k.shape[0] != B or k.shape[3] != D or v.shape != k.shape:
        raise ValueError("k, v must be [B, Sk, Hkv, D] matching q")
    Hkv = k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, Sq, Hq, D, k.shape[1], Hkv


def _scores(qh, kh, scale, causal, window=0):
    """scale * qh @ kh^T with the bottom-right causal mask (and the sliding
    window, if any) as -inf."""
    Sq, Sk = qh.shape[0], kh.shape[0]
    s = np.float64(scale) * (qh @ kh.T)
    if causal:
        pos = np.arange(Sq)[:, None] + (Sk - Sq)   # absolute position of each query
        j = np.arange(Sk)[None, :]
        s = np.where(j > pos, -np.inf, s)
        if window > 0:
            s = np.where(j <= pos - window, -np.inf, s)
    elif window > 0:
        raise ValueError("a sliding window needs causal attention")
    return s


def _softmax_rows(s):
    """Row softmax; rows with no finite score become all-zero rows."""
    m = np.max(s, axis=1, keepdims=True)
    dead = ~np.isfinite(m)
    m = np.where(dead, 0.0, m)
    p = np.exp(s - m)
    tot = np.sum(p, axis=1, keepdims=True)
    tot = np.where(dead, 1.0, tot)
    return p / tot


def attention_probs(q, k, scale, causal, b, h):
    """The [Sq, Sk] weight matrix of batch b, query head h (debug/pin use)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    G = q.shape[2] // k.shape[2]
    return _softmax_rows(_scores(q[b, :, h, :], k[b, :, h // G, :], scale, causal))


def attention(q, k, v, causal, scale, heads=None, window=0, mask=None):
    """out[b, i, h, :] = sum_j softmax_j(scale q_i.k_j + mask_ij) v_j.

    q [B,Sq,Hq,D], k/v [B,Sk,Hkv,D] (any float dtype; upcast to float64).
    ``heads`` optionally restricts the work to a list of (b, h) pairs; the
    other rows of the result are left as NaN.  ``window`` > 0 adds the
    sliding window (causal only).  ``mask`` [B, Hm, Sq, Sk] (Hm = 1 or Hq), if
    given, is added to the scaled scores on top of the causal mask.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Sq, Hq, D, Sk, Hkv = _check(q, k, v)
    G = Hq // Hkv
    if mask is not None:
        mask = np.asarray(mask, dtype=np.float64)
        if mask.ndim != 4 or mask.shape[0] != B or mask.shape[1] not in (1, Hq) or mask.shape[2:] != (Sq, Sk):
            raise ValueError("mask must be [B, 1 or Hq, Sq, Sk]")
    out = np.full((B, Sq, Hq, D), np.nan)
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    for b, h in pairs:
        kh = h // G
        s = _scores(q[b, :, h, :], k[b, :, kh, :], scale, causal, window)
        if mask is not None:
            s = s + mask[b, h if mask.shape[1] > 1 else 0]
        p = _softmax_rows(s)
        out[b, :, h, :] = p @ v[b, :, kh, :]
    return out


def attention_cache(q, k_cache, v_cache, kv_lens, causal, scale, window=0, heads=None):
    """Chunked / variable-length prefill against a cache.

    q [B,Sq,Hq,D]; caches [B,Hkv,max_kv,D] holding kv_len_b (clamped to
    [0, max_kv]) rotated rows per sequence.  Query i of sequence b sits at
    absolute position kv_len_b - Sq + i; with ``causal`` it sees keys
    j <= that position (and, with ``window`` W > 0, j > position - W); rows
    that see no key are zeros.  Sq = 1 is decode; Sq = kv_len is a plain
    prefill.  Returns float64 [B,Sq,Hq,D]; rows of pairs not in ``heads`` are
    NaN when ``heads`` is given.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Sq, Hq, D = q.shape
    _, Hkv, max_kv, _ = k_cache.shape
    G = Hq // Hkv
    out = np.full((B, Sq, Hq, D), np.nan)
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    for b, h in pairs:
        L = int(min(max(int(kv_lens[b]), 0), max_kv))
        kh = h // G
        if L == 0:
            out[b, :, h, :] = 0.0
            continue
        kk = np.asarray(k_cache[b, kh, :L, :], dtype=np.float64)
        vv = np.asarray(v_cache[b, kh, :L, :], dtype=np.float64)
        p = _softmax_rows(_scores(q[b, :, h, :], kk, scale, causal, window))
        out[b, :, h, :] = p @ vv
    return out


def decode(q, k_cache, v_cache, kv_lens, scale):
    """Single-token decode: q [B,Hq,D] against caches [B,Hkv,max_kv,D].

    Sequence b attends to cache rows 0 .. kv_len_b - 1 (kv_len clamped to
    [0, max_kv]); the cache already holds rotated keys, so nothing is rotated
    here.  Returns float64 [B, Hq, D].
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    _, Hkv, max_kv, _ = k_cache.shape
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    for b in range(B):
        L = int(min(max(int(kv_lens[b]), 0), max_kv))
        if L == 0:
            continue
        for kh in range(Hkv):
            kk = np.asarray(k_cache[b, kh, :L, :], dtype=np.float64)
            vv = np.asarray(v_cache[b, kh, :L, :], dtype=np.float64)
            qg = q[b, kh * G:(kh + 1) * G, :]           # the G query heads of this group
            p = _softmax_rows(_scores(qg, kk, scale, causal=False))
            out[b, kh * G:(kh + 1) * G, :] = p @ vv
    return out


def kv_append(k_cache, v_cache, k_new, v_new, slots):
    """Cache update: write k_new/v_new [B,Hkv,D] at row slots[b] of each cache.

    The cache grows along the sequence axis ("LLaMA2大语言模型架构详解",
    section "KV cache"); rows outside [0, max_kv) are not written.
    Returns updated float64 copies.
    """
    kc = np.array(k_cache, dtype=np.float64)
    vc = np.array(v_cache, dtype=np.float64)
    for b in range(kc.shape[0]):
        s = int(slots[b])
        if 0 <= s < kc.shape[2]:
            kc[b, :, s, :] = k_new[b]
            vc[b, :, s, :] = v_new[b]
    return kc, vc
