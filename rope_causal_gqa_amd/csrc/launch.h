// Internal launchers (host side) of librcgqa; arguments are validated by the
// C-ABI layer before any of these is called.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rcgqa {

// Where a prefill kernel finds the keys and values of (batch b, KV head g)
// and how many there are.  Element strides: row j of (b, g) starts at
// b*sb + g*sh + j*sr.  `lens` (device, may be null) holds each sequence's key
// count, clamped to [0, max_kv]; null means Sk = Sq.  Query i of a sequence
// with Sk keys sits at absolute position i + Sk - Sq; with a causal mask it
// sees keys j <= that position and, when window > 0, only j > position - window.
//
// mask (plain layout only; null = none): an additive mask of the run's element
// type, entry (b, h, i, j) at mask[b*msb + h*msh + i*msr + j], added to the
// scaled scores of query i and key j (msh = 0: shared by all query heads).
struct KvSpec {
  long long sb, sh, sr;
  const int32_t* lens;
  int max_kv;
  int window;
  const void* mask;
  long long msb, msh, msr;
};

// q may be null with Hq == 0 (keys only).  table, when not null, receives each
// token's fp32 cos/sin row ([B*S, D]: cos of pairs 0..D/2-1, then sin).
hipError_t launch_rope(void* q, void* k, const int32_t* pos, int B, int S, int Hq, int Hkv, int D,
                       double theta, double factor, bool bf16, float* table, hipStream_t st);
// Same contract with the interleaved pairing (x[2i], x[2i+1]).
hipError_t launch_rope_interleaved(void* q, void* k, const int32_t* pos, int B, int S, int Hq, int Hkv, int D,
                                  double theta, double factor, bool bf16_io, hipStream_t st);

// One decode step: rotate q into q_out and k_new at position pos[b] (kv_lens[b] - 1 when pos is null),
// append the rotated key and v_new at row kv_lens[b] - 1 of the caches.
hipError_t launch_rope_append(const void* q, void* q_out, const void* k_new, const void* v_new, void* k_cache,
                              void* v_cache, const int32_t* kv_lens, const int32_t* pos, int B, int Hq, int Hkv,
                              int D, int max_kv, double theta, double factor, bool bf16, hipStream_t st);

// q_rope, when not null, is the cos/sin table written by launch_rope for the
// queries' tokens ([B*Sq, D]); the kernels then rotate each query row as they
// load it, exactly as rope_apply would have.
hipError_t launch_prefill_f32(const float* q, const float* k, const float* v, float* out, int B, int Sq,
                              int Hq, int Hkv, int D, bool causal, float scale, const KvSpec& kv,
                              const float* q_rope, hipStream_t st);

hipError_t launch_prefill_bf16(const void* q, const void* k, const void* v, void* out, int B, int Sq,
                               int Hq, int Hkv, int D, bool causal, float scale, const KvSpec& kv,
                               const float* q_rope, hipStream_t st);

// Stream-K prefill for small causal grids without a cache or a mask (see
// grid::stream_plan): each workgroup runs an equal-cost range of (query
// tile, key tile) steps; pieces of a query tile shared by several
// workgroups write fp32 partial states to `ws` and the last one merges them.
// prefill_split_workspace_bytes is what `ws` must hold for these sizes (0 when
// the problem takes the one-workgroup-per-tile grids).  Its first 4 KB hold
// the per-tile counters of every shape: they must be zero before the first
// call, and every call leaves them zero.  Falls back to launch_prefill_bf16
// when the split is not used.
size_t prefill_split_workspace_bytes(int B, int Sq, int Hq, int D, bool causal);
// The same for a prefill of Sq query rows against a cache of max_kv rows
// (launch_prefill_bf16_split with kv.lens set).
size_t prefill_cache_split_workspace_bytes(int B, int Sq, int Hq, int D, int max_kv, bool causal, int window);
hipError_t launch_prefill_bf16_split(const void* q, const void* k, const void* v, void* out, int B, int Sq, int Hq,
                                     int Hkv, int D, bool causal, float scale, const KvSpec& kv, void* ws,
                                     hipStream_t st);

// Split-K decode: partial softmax states go to `ws`, then a merge pass writes out.
size_t decode_workspace_bytes(int B, int Hq, int D, int max_kv);
hipError_t launch_decode(const void* q, const void* kc, const void* vc, const int32_t* kv_lens, void* out,
                         int B, int Hq, int Hkv, int D, int max_kv, float scale, bool bf16, void* ws,
                         hipStream_t st);

// The no-allocation decode: partial states in a fixed per-device array of
// kDecodeNoAllocBytes.  decode_scratch_bytes is what launch_decode uses of a
// workspace for these sizes and element type; decode_noalloc_scratch returns
// the current device's array (looked up once per device).
constexpr size_t kDecodeNoAllocBytes = (size_t)16 << 20;
size_t decode_scratch_bytes(int B, int Hq, int D, int max_kv, bool bf16_io);
hipError_t decode_noalloc_scratch(void** ptr);

hipError_t launch_kv_append(void* kc, void* vc, const void* kn, const void* vn, const int32_t* slots, int B,
                            int Hkv, int D, int max_kv, bool bf16, hipStream_t st);

}  // namespace rcgqa
