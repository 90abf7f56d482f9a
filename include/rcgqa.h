/*
 * rcgqa.h -- C ABI of librcgqa: rotary position embedding and causal
 * grouped-query scaled-dot-product attention (prefill and single-token decode
 * against a KV cache) on AMD MI355X (gfx950).
 *
 * Sources (titles and sections of the pages the method is taken from):
 *   [HF]   "【HuggingFace Transformers】LlamaAttention源码解析" -- section 1.2 (attention
 *          steps 1-5), section 2 (LlamaAttention.forward, steps 1-6), section 3.1
 *          (LlamaFlashAttention2: variable lengths, mask alignment).
 *   [L2]   "LLaMA2大语言模型架构详解" -- sections "Rotary Position Encoding", "KV cache",
 *          "Grouped Multi-Query Attention (GQA)".
 *   [L2X]  "Llama2 Transformer架构解析与优化实践" -- sections 2.1, 3.2, 6.1.
 *   [VERL] "llama.py — LLaMA 注意力层 Ulysses SP 适配" -- "Ulysses SP 核心流程", step 2
 *          ("第二步：RoPE + Flash Attention", including its sliding_window argument).
 *   [TP]   "LLM Lab 实验手记 05：注意力张量并行" -- sections 2 and 5.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     allocates nothing and frees nothing.  Its only mutable state is a
 *     per-thread memo of the last prefill grid choice (a pure function of the
 *     shape) and, for attn_decode_noalloc only, a fixed 16 MiB device array per
 *     GPU with its address cached per device; calls from several threads are
 *     safe except overlapping attn_decode_noalloc calls on one GPU.
 *   - Tensors are dense and row-major with head_dim innermost.  Element type is
 *     selected by `dt`: RCGQA_BF16 (bfloat16 storage, fp32 arithmetic) or
 *     RCGQA_FP32.  Tensor pointers must be 16-byte aligned (the kernels move
 *     16-byte vectors) and int32 arrays 4-byte aligned; any device allocator's
 *     blocks are.  A misaligned pointer is RCGQA_EINVAL.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream).  Nothing synchronises inside the library.
 *   - Errors: every argument that can be checked on the host is checked before
 *     any launch; a bad one returns RCGQA_EINVAL and launches nothing.  A shape
 *     the kernels do not implement returns RCGQA_EUNSUPPORTED.  A failed launch
 *     returns RCGQA_EHIP.  Device-resident values (positions, kv_lens) are not
 *     read on the host; the kernels clamp them as documented per call.
 *   - Sizes are int; the element count of every tensor must fit in int64 and
 *     B*S (and B*Hq) must fit in int32.
 *   - Grid limits (RCGQA_EUNSUPPORTED): the prefill entry points take at most
 *     4194240 query rows per sequence and B*Hq*ceil(S/128) <= 2^24 - 1 (about
 *     2^31 query rows in all, more than q and out could fill in one GPU's
 *     memory); the decode entry points and kv_append at most 65535 sequences
 *     and 65535 heads.
 */
#ifndef RCGQA_H
#define RCGQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RCGQA_OK = 0,
  RCGQA_EINVAL = 1,       /* bad argument (checked on the host, nothing launched) */
  RCGQA_EUNSUPPORTED = 2, /* valid, but no kernel for this head_dim / dtype       */
  RCGQA_EHIP = 3,         /* the HIP runtime reported an error at launch          */
  RCGQA_ENOSPACE = 4      /* too large for the fixed scratch of attn_decode_noalloc */
} rcgqa_status;

typedef enum { RCGQA_BF16 = 0, RCGQA_FP32 = 1 } rcgqa_dtype;

/* A hipStream_t passed as an opaque pointer; NULL selects the null stream. */
typedef void* rcgqa_stream;

/*
 * rope_apply -- rotate queries and keys in place by their positions.
 *
 * Defines: [L2] "Rotary Position Encoding" (RoFormer rotation; applied to Q
 * and K only, after projection, never to V); [HF] section 2 step 3
 * (apply_rotary_pos_emb with cos/sin from rope_theta and position_ids);
 * [L2X] section 6.1 (linear rope_scaling factor).
 *
 *   pair i of every head vector, i in [0, head_dim/2), is (x[i], x[i+head_dim/2])
 *   angle = (pos / linear_factor) * theta^(-2 i / head_dim)
 *   (x1, x2) <- (x1 cos(angle) - x2 sin(angle), x2 cos(angle) + x1 sin(angle))
 *
 * q            [B, S, Hq,  head_dim]  in/out
 * k            [B, S, Hkv, head_dim]  in/out
 * position_ids [B, S] int32 device array, or NULL for 0..S-1 in every sequence.
 *              Any int32 value is accepted (negative positions rotate backwards).
 * theta        RoPE base (> 0, finite), e.g. 10000.
 * linear_factor positions are divided by it (> 0, finite); 1 = no scaling.
 * head_dim     even, 2..256.
 * Angles are formed in fp64 and their cos/sin rounded to fp32; the rotation is
 * computed in fp32 and, for bf16, rounded once to bf16 (nearest even).
 */
rcgqa_status rope_apply(void* q, void* k, const int32_t* position_ids,
                        int B, int S, int Hq, int Hkv, int head_dim,
                        float theta, float linear_factor,
                        rcgqa_dtype dt, rcgqa_stream stream);

/*
 * rope_apply_interleaved -- rope_apply with adjacent pairs.
 *
 * Defines: the same rotation as rope_apply ([L2] "Rotary Position Encoding";
 * [L2X] sections 2.1 and 6.1), with the pairing of its complex-number form
 * ([L2X] section 2.1 calls it a rotation in the complex domain): element pair
 * i is (x[2i], x[2i+1]), i.e. a fixed permutation of the head dimension away
 * from rope_apply's (x[i], x[i+head_dim/2]).
 *
 *   pair i of every head vector, i in [0, head_dim/2), is (x[2i], x[2i+1])
 *   angle = (pos / linear_factor) * theta^(-2 i / head_dim)
 *   (x1, x2) <- (x1 cos(angle) - x2 sin(angle), x2 cos(angle) + x1 sin(angle))
 *
 * Arguments, layouts, precision and errors exactly as rope_apply; for every
 * pair the angle, cos/sin and arithmetic are rope_apply's, so permuting the
 * head dimension maps one result onto the other bit for bit.
 */
rcgqa_status rope_apply_interleaved(void* q, void* k, const int32_t* position_ids,
                                    int B, int S, int Hq, int Hkv, int head_dim,
                                    float theta, float linear_factor,
                                    rcgqa_dtype dt, rcgqa_stream stream);

/*
 * rope_ntk_theta / rope_dynamic_ntk_theta -- the RoPE base for NTK-aware
 * scaling (host-side arithmetic; nothing is launched).
 *
 * Defines: [L2X] section 6.1 names NTK-aware scaling, next to linear
 * interpolation, as a way to extend RoPE past the trained length by adjusting
 * the rotation angles; it prints no formula.  The definition taken is the
 * published "NTK-aware scaled RoPE" one (2023; also the dynamic NTK rotary
 * embedding of Hugging Face Transformers): positions are not divided, the base
 * is raised instead so that the highest-frequency pair keeps its angle and
 * the lowest-frequency pair is divided by the scale alpha:
 *
 *   theta_out = theta * alpha^(head_dim / (head_dim - 2))
 *
 * The dynamic form takes alpha = factor * seq_len / max_position - (factor - 1)
 * when seq_len > max_position, and returns theta unchanged otherwise.  Pass
 * theta_out (with linear_factor 1) to rope_apply or the fused entry points.
 *
 * theta > 0, finite; head_dim even, >= 4; alpha > 0, finite; factor > 0,
 * finite; seq_len, max_position >= 1; theta_out non-null.  The value is
 * formed in double and rounded once to float; a result that is not a finite
 * float is RCGQA_EINVAL.
 */
rcgqa_status rope_ntk_theta(float theta, int head_dim, float alpha, float* theta_out);
rcgqa_status rope_dynamic_ntk_theta(float theta, int head_dim, float factor, int seq_len,
                                    int max_position, float* theta_out);

/*
 * attn_prefill -- full-sequence scaled-dot-product attention, grouped-query.
 *
 * Defines: [HF] section 1.2 steps 2-4 and section 2 steps 4-5 (scores
 * Q K^T * scale, additive causal mask, fp32 softmax, weights @ V); the
 * grouped-query head map of repeat_kv ([HF] section 2 step 4; [L2] GQA;
 * [L2X] section 2.1): query head h reads K/V head h / (Hq/Hkv).
 *
 *   out[b,i,h,:] = sum_j softmax_j(scale * q[b,i,h,:].k[b,j,h/G,:] + mask_ij) v[b,j,h/G,:]
 *   mask_ij = -inf where causal and j > i, else 0.
 *
 * q   [B, S, Hq,  head_dim]
 * k,v [B, S, Hkv, head_dim]
 * out [B, S, Hq,  head_dim]  (= [B, S, Hq*head_dim], the merged-heads layout)
 * causal  0 or 1.   scale > 0, finite (usually 1/sqrt(head_dim)).
 * Hq % Hkv == 0.  head_dim: 64 or 128 (bf16 and fp32).
 * Scores and softmax state are fp32; for bf16 the softmax weights are rounded
 * to bf16 as the P@V operand, accumulation is fp32 and out is rounded to bf16.
 * out must not alias q, k or v.
 */
rcgqa_status attn_prefill(const void* q, const void* k, const void* v, void* out,
                          int B, int S, int Hq, int Hkv, int head_dim,
                          int causal, float scale,
                          rcgqa_dtype dt, rcgqa_stream stream);

/*
 * attn_prefill_workspace_bytes -- bytes of scratch attn_prefill_ws needs for
 * these sizes.  Pure host function.  0 when the problem runs without one (see
 * attn_prefill_ws: large, short or not causal); returns 0 if an argument is
 * not positive.
 */
size_t attn_prefill_workspace_bytes(int B, int S, int Hq, int head_dim, int causal);

/*
 * attn_prefill_ws -- attn_prefill with a caller-owned workspace, which lets
 * small causal problems spread each query tile's keys over several
 * workgroups.
 *
 * Defines: as attn_prefill ([HF] section 1.2 steps 2-4 and section 2 steps
 * 4-5; repeat_kv head map).  For a causal bf16 problem too small to fill the
 * GPU with pairs of heavy and light query tiles (for example one GPU's
 * 8-query-head / 1-KV-head share of a 64-head layer, the head split of [L2X]
 * section 3.1, or 16 query heads of 4096 tokens) but with at least 4096
 * (256-row query tile, 64-key tile) steps, the steps are cut into 256
 * contiguous ranges of equal cost, one per workgroup, which may cross query
 * tiles (stream-K).  A query tile shared by
 * several workgroups is finished by the last of them to end: each writes its
 * softmax state (fp32 O, running max, row sum) to the workspace, and the
 * last merges the states in key order, so the result is repeatable bit for
 * bit.  Other problems (large, short, non-causal, longer than 32768 tokens,
 * fp32) run exactly as attn_prefill.
 *
 * Arguments as attn_prefill, plus:
 * workspace  device buffer of at least attn_prefill_workspace_bytes(B, S, Hq,
 *            head_dim, causal) bytes (may be null when that is 0), 256-byte
 *            aligned, owned by the caller.  Its first 4096 bytes hold per-tile
 *            counters and must be zero before its first use (for example
 *            hipMemset of the whole buffer); every call leaves them zero, so
 *            one workspace serves later calls of any shape it is large
 *            enough for.  Concurrent calls must not share a workspace.
 * Errors as attn_prefill; a workspace that is too small, misaligned or null
 * when needed is RCGQA_EINVAL (nothing launched).
 */
rcgqa_status attn_prefill_ws(const void* q, const void* k, const void* v, void* out,
                             int B, int S, int Hq, int Hkv, int head_dim,
                             int causal, float scale, rcgqa_dtype dt,
                             void* workspace, size_t workspace_bytes,
                             rcgqa_stream stream);

/*
 * attn_prefill_masked -- attn_prefill with a general additive mask.
 *
 * Defines: [HF] section 1.2 step 3 (the attention mask is sliced to the query
 * and key lengths and added to the scaled scores before the fp32 softmax) and
 * section 2 steps 4-5, for any mask: padding, per-head biases, custom
 * patterns.  The causal mask can be applied on top.
 *
 *   out[b,i,h,:] = sum_j softmax_j(scale * q[b,i,h,:].k[b,j,h/G,:] + mask[b,h',i,j]
 *                                  + (causal && j > i ? -inf : 0)) v[b,j,h/G,:]
 *   h' = 0 when mask_heads == 1 (one mask shared by all query heads), else h.
 *
 * q, k, v, out  as attn_prefill ([B,S,Hq|Hkv,head_dim], head_dim 64 or 128).
 * mask  [B, mask_heads, S, mask_ld] of the run's element type, row stride
 *       mask_ld >= S elements (entries j >= S of a row are not read), 16-byte
 *       aligned base; mask_heads is 1 or Hq.  -inf entries give zero weight; a
 *       row with no finite score returns zeros.  Entries are added in fp32 to
 *       the fp32 scores (bf16 masks are read exactly).
 * out must not alias q, k, v or mask.
 */
rcgqa_status attn_prefill_masked(const void* q, const void* k, const void* v, const void* mask, void* out,
                                 int B, int S, int Hq, int Hkv, int head_dim,
                                 int mask_heads, int mask_ld, int causal, float scale,
                                 rcgqa_dtype dt, rcgqa_stream stream);

/*
 * attn_prefill_cache -- chunked / variable-length prefill against a KV cache,
 * with an optional causal sliding window.
 *
 * Defines: [HF] section 1.2 steps 2-4 and section 2 steps 4-5 (scores, mask,
 * fp32 softmax, weights @ V, repeat_kv head map) for a block of Sq new query
 * tokens per sequence whose keys and values, together with all earlier ones,
 * are in the cache ([L2] "KV cache"; [HF] section 3.1: variable-length
 * sequences, and the mask aligned to the end of the key range, the
 * use_top_left_mask alternative being the other alignment).  The sliding
 * window is the one the flash-attention call of [VERL] "第二步：RoPE + Flash
 * Attention" passes; the pages do not define it, so the reading is: the
 * query at absolute position p sees only keys p - window < j <= p.
 *
 *   L_b = clamp(kv_lens[b], 0, max_kv);  query i of sequence b is at p = L_b - Sq + i
 *   out[b,i,h,:] = sum_{j in K(b,i)} softmax_j(scale * q[b,i,h,:].K[b,h/G,j,:]) V[b,h/G,j,:]
 *   K(b,i) = { j < L_b }                                   causal == 0
 *          = { j <= p }                                    causal == 1, window == 0
 *          = { p - window < j <= p }                       causal == 1, window > 0
 *   A row with an empty K(b,i) (p < 0, or L_b == 0) is a zero row.
 *
 * q        [B, Sq, Hq, head_dim]          (already rotated)
 * k_cache  [B, Hkv, max_kv, head_dim]     rows 0..L_b-1 valid, already rotated;
 *                                         the last Sq of them are this block's own keys
 * v_cache  [B, Hkv, max_kv, head_dim]
 * kv_lens  [B] int32 device array (not read on the host; clamped by the kernels)
 * out      [B, Sq, Hq, head_dim]
 * causal 0 or 1; window >= 0 (0 = none; window > 0 needs causal == 1).
 * scale > 0, finite.  Hq % Hkv == 0.  head_dim: 64 or 128 (bf16 and fp32).
 * Sq == 1 is a decode step (attn_decode is the faster kernel for it); Sq ==
 * L_b for every b is a plain prefill.  Numerics as attn_prefill.  out must not
 * alias q or the caches.
 */
rcgqa_status attn_prefill_cache(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* kv_lens, void* out,
                                int B, int Sq, int Hq, int Hkv, int head_dim, int max_kv,
                                int causal, int window, float scale,
                                rcgqa_dtype dt, rcgqa_stream stream);

/*
 * attn_prefill_cache_workspace_bytes -- bytes of scratch attn_prefill_cache_ws
 * needs for these sizes.  Pure host function.  0 when the problem runs
 * without one (see attn_prefill_cache_ws); 0 if an argument is not positive.
 */
size_t attn_prefill_cache_workspace_bytes(int B, int Sq, int Hq, int head_dim, int max_kv, int causal,
                                          int window);

/*
 * attn_prefill_cache_ws -- attn_prefill_cache with a caller-owned workspace,
 * which lets causal chunks without a window spread their work over all
 * workgroups.
 *
 * Defines: as attn_prefill_cache ([HF] section 1.2 steps 2-4 and section 2
 * steps 4-5 over the cached keys; [L2] "KV cache").  For a causal bf16 block
 * with no window, max_kv >= Sq, and too few query tiles to fill the GPU with
 * pairs of them (for example a chunk of 512 new tokens after 4096 cached
 * ones), the work is listed as (256-row query tile, 64-key tile) steps,
 * counted as if every sequence held max_kv rows, and cut into 256 contiguous
 * ranges of equal cost, one per workgroup (stream-K, as attn_prefill_ws).
 * Shorter sequences are still exact: the steps past their keys are skipped.
 * A query tile shared by several workgroups is merged by the last of them in
 * key order, so the result repeats bit for bit.  Other problems run exactly
 * as attn_prefill_cache.
 *
 * Arguments as attn_prefill_cache, plus workspace / workspace_bytes with the
 * contract of attn_prefill_ws (at least attn_prefill_cache_workspace_bytes
 * bytes, 256-byte aligned, its first 4096 bytes zero before the first use
 * and left zero by every call; not shared by concurrent calls).  Errors as
 * attn_prefill_cache; a workspace that is too small, misaligned, null when
 * needed or equal to another argument is RCGQA_EINVAL (nothing launched).
 */
rcgqa_status attn_prefill_cache_ws(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* kv_lens, void* out,
                                   int B, int Sq, int Hq, int Hkv, int head_dim, int max_kv,
                                   int causal, int window, float scale, rcgqa_dtype dt,
                                   void* workspace, size_t workspace_bytes, rcgqa_stream stream);

/*
 * attn_decode_workspace_bytes -- bytes of scratch attn_decode needs for these
 * sizes (partial softmax states of the split-K pass).  Pure host function.
 * Returns 0 if an argument is not positive.
 */
size_t attn_decode_workspace_bytes(int B, int Hq, int head_dim, int max_kv);

/*
 * attn_decode -- one new query token per sequence against a KV cache.
 *
 * Defines: [L2] "KV cache" (the new token's query attends to all cached keys
 * and itself; earlier rows are not recomputed) and "Grouped Multi-Query
 * Attention" (one K/V stream serves the G query heads of its group);
 * [HF] section 2 steps 3-5 (keys are cached after rotation).
 *
 *   out[b,h,:] = sum_{j < L_b} softmax_j(scale * q[b,h,:].K[b,h/G,j,:]) V[b,h/G,j,:]
 *   L_b = clamp(kv_lens[b], 0, max_kv);  L_b == 0 gives a zero row.
 *
 * q        [B, Hq, head_dim]            (already rotated)
 * k_cache  [B, Hkv, max_kv, head_dim]   rows 0..L_b-1 valid, already rotated
 * v_cache  [B, Hkv, max_kv, head_dim]
 * kv_lens  [B] int32 device array
 * out      [B, Hq, head_dim]
 * workspace  device buffer of at least attn_decode_workspace_bytes(B, Hq,
 *            head_dim, max_kv) bytes, 256-byte aligned, owned by the caller;
 *            no initial contents are required.  Concurrent calls must not
 *            share a workspace.
 * head_dim: 64 or 128.  Hq % Hkv == 0, Hq/Hkv <= 16.  out must not alias q or
 * the caches.
 * The result does not depend on the order in which partial states finish:
 * partial states are merged in a fixed order (bitwise repeatable).
 */
rcgqa_status attn_decode(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* kv_lens, void* out,
                         int B, int Hq, int Hkv, int head_dim, int max_kv,
                         float scale, rcgqa_dtype dt,
                         void* workspace, size_t workspace_bytes,
                         rcgqa_stream stream);

/*
 * attn_decode_noalloc -- attn_decode without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, serving
 * loops, harnesses that forbid allocation).  Same arguments, result and
 * kernels as attn_decode (bit-identical output); the split-K partial states
 * go to a fixed array of 16 MiB that the library holds on every GPU it runs
 * on until the process ends.  The call itself allocates and frees nothing.
 *
 * Limit: the partial states must fit in 16 MiB, i.e.
 *   B * Hq * ceil(max_kv / 2048) * (head_dim + 2) * 4 bytes for RCGQA_BF16,
 *   B * Hq * ceil(max_kv / 256)  * (head_dim + 2) * 4 bytes for RCGQA_FP32;
 * larger problems return RCGQA_ENOSPACE and launch nothing (the B=64 Hq=64
 * head_dim=128 max_kv=8193 bf16 decode needs 10.6 MB).  The array needs no
 * initial contents and every call overwrites what it reads.
 * The array is found for the calling thread's current device (hipGetDevice),
 * so `stream` must belong to that device.  All calls on one GPU share its
 * array: calls that overlap in time on one GPU (different streams or threads)
 * race and give wrong results; serialise them, or use attn_decode with
 * separate workspaces.
 */
rcgqa_status attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* kv_lens, void* out,
                                 int B, int Hq, int Hkv, int head_dim, int max_kv,
                                 float scale, rcgqa_dtype dt, rcgqa_stream stream);

/*
 * kv_append -- write one new key row and value row per sequence into the cache.
 *
 * Defines: [L2] "KV cache" (K and V grow by appending the new token's row);
 * [HF] section 2 step 3 (past_key_value.update after the rotation).
 *
 * k_new, v_new [B, Hkv, head_dim]; caches [B, Hkv, max_kv, head_dim];
 * slots [B] int32 device array: row written for sequence b.  A slot outside
 * [0, max_kv) writes nothing for that sequence.  head_dim even, <= 256.
 */
rcgqa_status kv_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                       const int32_t* slots, int B, int Hkv, int head_dim, int max_kv,
                       rcgqa_dtype dt, rcgqa_stream stream);

/*
 * rope_attn_prefill_workspace_bytes -- bytes of scratch rope_attn_prefill
 * needs: one fp32 cos/sin row per token, B * S * head_dim * 4.  Pure host
 * function; 0 if an argument is not positive or the size overflows.
 */
size_t rope_attn_prefill_workspace_bytes(int B, int S, int head_dim);

/*
 * rope_attn_prefill -- rope_apply followed by attn_prefill, with the query
 * rotation done inside the attention kernel as each query row is loaded.
 *
 * Defines: the composition of rope_apply and attn_prefill above ([L2]
 * "Rotary Position Encoding"; [HF] section 2 steps 3-5: rotate Q and K, then
 * attention; [L2X] section 6.1 for linear_factor).  The result is the one the
 * two separate calls produce, bit for bit: the keys are rotated by the same
 * kernel, and each query row is rotated with the same fp32 cos/sin values and
 * the same arithmetic and rounding before it enters the score products.
 *
 * q            [B, S, Hq,  head_dim]  read only: NOT rotated in memory
 * k            [B, S, Hkv, head_dim]  in/out: rotated in place, as rope_apply
 *                                     leaves it (the keys a KV cache keeps)
 * v            [B, S, Hkv, head_dim]
 * out          [B, S, Hq,  head_dim]
 * position_ids [B, S] int32 device array, or NULL for 0..S-1 in every sequence.
 * causal, scale, theta, linear_factor, Hq % Hkv, head_dim (64 or 128): as
 * rope_apply and attn_prefill.
 * workspace  device buffer of at least rope_attn_prefill_workspace_bytes(B, S,
 *            head_dim) bytes, 256-byte aligned, owned by the caller; no initial
 *            contents are required; it holds the cos/sin rows and concurrent
 *            calls must not share it.
 * out must not alias q, k or v, and q, k, v must be distinct buffers.
 * Traffic: the rotation adds one read and one write of K (plus the small
 * table) to the attention pass, instead of a read and write of Q and K.
 */
rcgqa_status rope_attn_prefill(const void* q, void* k, const void* v, void* out,
                               const int32_t* position_ids,
                               int B, int S, int Hq, int Hkv, int head_dim,
                               int causal, float scale, float theta, float linear_factor,
                               rcgqa_dtype dt, void* workspace, size_t workspace_bytes,
                               rcgqa_stream stream);

/*
 * rope_attn_decode_workspace_bytes -- bytes of scratch rope_attn_decode needs
 * (the rotated queries, then attn_decode's split-K partial states).  Pure host
 * function; 0 if an argument is not positive.
 */
size_t rope_attn_decode_workspace_bytes(int B, int Hq, int head_dim, int max_kv);

/*
 * rope_attn_decode -- one decode step with the rotations and the cache append
 * fused into one kernel ahead of the decode attention.
 *
 * Defines: [L2] "KV cache" (the new token's key and value are appended, its
 * query attends to every cached key and itself) and "Rotary Position
 * Encoding"; [HF] section 2 steps 3-5 (q and the new key are rotated at the
 * token's position before the key is cached and attention runs).  Exactly
 * the composition, bit for bit:
 *   rope_apply(q, k_new at positions pos_b);
 *   kv_append(k_cache, v_cache, rotated k_new, v_new, slots = kv_lens - 1);
 *   attn_decode(rotated q, k_cache, v_cache, kv_lens, out)
 * with pos_b = position_ids[b], or kv_lens[b] - 1 when position_ids is NULL
 * (the new token sits right after the ctx = kv_lens[b] - 1 cached ones).
 *
 * q            [B, Hq, head_dim]   read only (not rotated in memory)
 * k_new, v_new [B, Hkv, head_dim]  read only
 * k_cache, v_cache [B, Hkv, max_kv, head_dim]  in/out: row kv_lens[b] - 1 is
 *              written with the rotated k_new / v_new (nothing is written for
 *              a sequence whose row is outside [0, max_kv))
 * kv_lens      [B] int32 device array: lengths INCLUDING the new token;
 *              attention uses clamp(kv_lens[b], 0, max_kv) as attn_decode.
 * position_ids [B] int32 device array, or NULL.
 * out          [B, Hq, head_dim]
 * workspace    at least rope_attn_decode_workspace_bytes(B, Hq, head_dim,
 *              max_kv) bytes, 256-byte aligned, caller-owned, no initial
 *              contents needed; concurrent calls must not share it.
 * head_dim 64 or 128; Hq % Hkv == 0, Hq/Hkv <= 16; scale, theta,
 * linear_factor > 0 and finite.
 */
rcgqa_status rope_attn_decode(const void* q, const void* k_new, const void* v_new,
                              void* k_cache, void* v_cache,
                              const int32_t* kv_lens, const int32_t* position_ids, void* out,
                              int B, int Hq, int Hkv, int head_dim, int max_kv,
                              float scale, float theta, float linear_factor,
                              rcgqa_dtype dt, void* workspace, size_t workspace_bytes,
                              rcgqa_stream stream);

/* Static, human-readable name of a status code. */
const char* rcgqa_status_string(rcgqa_status s);

#ifdef __cplusplus
}
#endif

#endif /* RCGQA_H */
