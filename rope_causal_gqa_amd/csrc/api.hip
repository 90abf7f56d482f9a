// C ABI of librcgqa (declared in include/rcgqa.h): host-side validation and
// dispatch to the gfx950 kernels.  Nothing here allocates, synchronises or
// keeps state; every check that can be made on the host is made before the
// first launch, so a rejected call launches nothing.
#include <cmath>
#include <cstdint>

#include "launch.h"
#include "rcgqa.h"

namespace {

constexpr int64_t kI32Max = 2147483647;

bool pos_int(int x) { return x >= 1; }
bool good_dtype(rcgqa_dtype dt) { return dt == RCGQA_BF16 || dt == RCGQA_FP32; }
bool finite_pos(float x) { return std::isfinite(x) && x > 0.f; }
// Tensors are accessed in 16-byte vectors (and 16-byte direct-to-LDS loads),
// int32 arrays element-wise; null pointers pass here and are rejected apart.
bool al16(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (reinterpret_cast<uintptr_t>(p) & 15) return false;
  return true;
}
bool al4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3) == 0; }

// Product of positive ints, or -1 on int64 overflow.
int64_t mul(std::initializer_list<int64_t> xs) {
  int64_t p = 1;
  for (int64_t x : xs) {
    if (x <= 0) return -1;
    if (p > INT64_MAX / x) return -1;
    p *= x;
  }
  return p;
}

bool attn_head_dim(int d) { return d == 64 || d == 128; }

// Grid limits of the prefill kernels.  Query rows of a sequence are tiled in
// at most 65535 blocks of 64 in the fp32 kernel's second grid dimension, and
// no prefill grid launches more than two work-items per query row once each
// (batch, head)'s rows are padded to a multiple of 128; a dispatch counts its
// work-items in 32 bits.  (2^32 work-items means about 2^31 query rows: q and
// out alone would not fit in one GPU's memory.)
bool prefill_grid_ok(int B, int Hq, int S) {
  if ((S + 63) / 64 > 65535) return false;
  const int64_t items = mul({B, Hq, (S + 127) / 128, 256});
  return items > 0 && items <= (int64_t)UINT32_MAX;
}

rcgqa_status hip_status(hipError_t e) { return e == hipSuccess ? RCGQA_OK : RCGQA_EHIP; }

// Host checks shared by the two pairings of the rotation.
rcgqa_status rope_check(const void* q, const void* k, int B, int S, int Hq, int Hkv, int head_dim, float theta,
                        float linear_factor, rcgqa_dtype dt) {
  if (!q || !k || !good_dtype(dt) || !al16({q, k})) return RCGQA_EINVAL;
  if (!pos_int(B) || !pos_int(S) || !pos_int(Hq) || !pos_int(Hkv) || Hq % Hkv) return RCGQA_EINVAL;
  if (head_dim < 2 || head_dim % 2) return RCGQA_EINVAL;
  if (!finite_pos(theta) || !finite_pos(linear_factor)) return RCGQA_EINVAL;
  const int64_t tokens = mul({B, S});
  if (tokens < 0 || tokens > kI32Max || mul({tokens, Hq, head_dim}) < 0) return RCGQA_EINVAL;
  if (head_dim > 256) return RCGQA_EUNSUPPORTED;
  return RCGQA_OK;
}

}  // namespace

extern "C" {

const char* rcgqa_status_string(rcgqa_status s) {
  switch (s) {
    case RCGQA_OK: return "ok";
    case RCGQA_EINVAL: return "invalid argument";
    case RCGQA_EUNSUPPORTED: return "unsupported head_dim or dtype";
    case RCGQA_EHIP: return "HIP runtime error at launch";
    case RCGQA_ENOSPACE: return "problem needs more than the library's fixed scratch (use the workspace entry point)";
  }
  return "unknown status";
}

rcgqa_status rope_apply(void* q, void* k, const int32_t* position_ids, int B, int S, int Hq, int Hkv,
                        int head_dim, float theta, float linear_factor, rcgqa_dtype dt, rcgqa_stream stream) {
  const rcgqa_status bad = rope_check(q, k, B, S, Hq, Hkv, head_dim, theta, linear_factor, dt);
  if (bad != RCGQA_OK) return bad;
  if (!al4(position_ids)) return RCGQA_EINVAL;
  return hip_status(rcgqa::launch_rope(q, k, position_ids, B, S, Hq, Hkv, head_dim, (double)theta,
                                       (double)linear_factor, dt == RCGQA_BF16, nullptr, (hipStream_t)stream));
}

rcgqa_status rope_apply_interleaved(void* q, void* k, const int32_t* position_ids, int B, int S, int Hq, int Hkv,
                                    int head_dim, float theta, float linear_factor, rcgqa_dtype dt,
                                    rcgqa_stream stream) {
  const rcgqa_status bad = rope_check(q, k, B, S, Hq, Hkv, head_dim, theta, linear_factor, dt);
  if (bad != RCGQA_OK) return bad;
  if (!al4(position_ids)) return RCGQA_EINVAL;
  return hip_status(rcgqa::launch_rope_interleaved(q, k, position_ids, B, S, Hq, Hkv, head_dim, (double)theta,
                                                   (double)linear_factor, dt == RCGQA_BF16, (hipStream_t)stream));
}

rcgqa_status rope_ntk_theta(float theta, int head_dim, float alpha, float* theta_out) {
  if (!theta_out || !finite_pos(theta) || !finite_pos(alpha) || head_dim < 4 || head_dim % 2) return RCGQA_EINVAL;
  const double t = (double)theta * std::pow((double)alpha, (double)head_dim / (double)(head_dim - 2));
  const float f = (float)t;
  if (!finite_pos(f)) return RCGQA_EINVAL;
  *theta_out = f;
  return RCGQA_OK;
}

rcgqa_status rope_dynamic_ntk_theta(float theta, int head_dim, float factor, int seq_len, int max_position,
                                    float* theta_out) {
  if (!theta_out || !finite_pos(theta) || !finite_pos(factor) || head_dim < 4 || head_dim % 2) return RCGQA_EINVAL;
  if (!pos_int(seq_len) || !pos_int(max_position)) return RCGQA_EINVAL;
  if (seq_len <= max_position) {
    *theta_out = theta;
    return RCGQA_OK;
  }
  const double alpha = (double)factor * (double)seq_len / (double)max_position - ((double)factor - 1.0);
  if (!(alpha > 0.0)) return RCGQA_EINVAL;
  const double t = (double)theta * std::pow(alpha, (double)head_dim / (double)(head_dim - 2));
  const float f = (float)t;
  if (!finite_pos(f)) return RCGQA_EINVAL;
  *theta_out = f;
  return RCGQA_OK;
}

rcgqa_status attn_prefill(const void* q, const void* k, const void* v, void* out, int B, int S, int Hq, int Hkv,
                          int head_dim, int causal, float scale, rcgqa_dtype dt, rcgqa_stream stream) {
  if (!q || !k || !v || !out || !good_dtype(dt) || !al16({q, k, v, out})) return RCGQA_EINVAL;
  if (out == q || out == k || out == v) return RCGQA_EINVAL;
  if (!pos_int(B) || !pos_int(S) || !pos_int(Hq) || !pos_int(Hkv) || Hq % Hkv) return RCGQA_EINVAL;
  if (head_dim < 2 || head_dim % 2 || (causal != 0 && causal != 1) || !finite_pos(scale)) return RCGQA_EINVAL;
  if (mul({B, Hq}) > kI32Max || mul({B, S, Hq, head_dim}) < 0) return RCGQA_EINVAL;
  if (!attn_head_dim(head_dim) || !prefill_grid_ok(B, Hq, S)) return RCGQA_EUNSUPPORTED;
  const hipStream_t st = (hipStream_t)stream;
  // K/V in [B, S, Hkv, D]: every sequence has S keys, queries aligned with them
  const rcgqa::KvSpec kv{(long long)S * Hkv * head_dim, head_dim, (long long)Hkv * head_dim, nullptr, S, 0};
  if (dt == RCGQA_BF16)
    return hip_status(
        rcgqa::launch_prefill_bf16(q, k, v, out, B, S, Hq, Hkv, head_dim, causal != 0, scale, kv, nullptr, st));
  return hip_status(rcgqa::launch_prefill_f32((const float*)q, (const float*)k, (const float*)v, (float*)out, B, S,
                                              Hq, Hkv, head_dim, causal != 0, scale, kv, nullptr, st));
}

size_t attn_prefill_workspace_bytes(int B, int S, int Hq, int head_dim, int causal) {
  if (!pos_int(B) || !pos_int(S) || !pos_int(Hq) || !pos_int(head_dim)) return 0;
  if (mul({B, Hq}) > kI32Max || !attn_head_dim(head_dim)) return 0;
  return rcgqa::prefill_split_workspace_bytes(B, S, Hq, head_dim, causal != 0);
}

rcgqa_status attn_prefill_ws(const void* q, const void* k, const void* v, void* out, int B, int S, int Hq, int Hkv,
                             int head_dim, int causal, float scale, rcgqa_dtype dt, void* workspace,
                             size_t workspace_bytes, rcgqa_stream stream) {
  if (!q || !k || !v || !out || !good_dtype(dt) || !al16({q, k, v, out})) return RCGQA_EINVAL;
  if (out == q || out == k || out == v) return RCGQA_EINVAL;
  if (!pos_int(B) || !pos_int(S) || !pos_int(Hq) || !pos_int(Hkv) || Hq % Hkv) return RCGQA_EINVAL;
  if (head_dim < 2 || head_dim % 2 || (causal != 0 && causal != 1) || !finite_pos(scale)) return RCGQA_EINVAL;
  if (mul({B, Hq}) > kI32Max || mul({B, S, Hq, head_dim}) < 0) return RCGQA_EINVAL;
  if (!attn_head_dim(head_dim) || !prefill_grid_ok(B, Hq, S)) return RCGQA_EUNSUPPORTED;
  const size_t need = dt == RCGQA_BF16 ? attn_prefill_workspace_bytes(B, S, Hq, head_dim, causal) : 0;
  if (need && (!workspace || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % 256))
    return RCGQA_EINVAL;
  if (workspace && (workspace == q || workspace == k || workspace == v || workspace == out)) return RCGQA_EINVAL;
  const hipStream_t st = (hipStream_t)stream;
  const rcgqa::KvSpec kv{(long long)S * Hkv * head_dim, head_dim, (long long)Hkv * head_dim, nullptr, S, 0};
  if (dt == RCGQA_BF16)
    return hip_status(rcgqa::launch_prefill_bf16_split(q, k, v, out, B, S, Hq, Hkv, head_dim, causal != 0, scale, kv,
                                                       need ? workspace : nullptr, st));
  return hip_status(rcgqa::launch_prefill_f32((const float*)q, (const float*)k, (const float*)v, (float*)out, B, S,
                                              Hq, Hkv, head_dim, causal != 0, scale, kv, nullptr, st));
}

size_t attn_prefill_cache_workspace_bytes(int B, int Sq, int Hq, int head_dim, int max_kv, int causal, int window) {
  if (!pos_int(B) || !pos_int(Sq) || !pos_int(Hq) || !pos_int(head_dim) || !pos_int(max_kv) || window < 0) return 0;
  if (mul({B, Hq}) > kI32Max || !attn_head_dim(head_dim)) return 0;
  if (window >= max_kv) window = 0;
  return rcgqa::prefill_cache_split_workspace_bytes(B, Sq, Hq, head_dim, max_kv, causal != 0, window);
}

rcgqa_status attn_prefill_cache_ws(const void* q, const void* k_cache, const void* v_cache, const int32_t* kv_lens,
                                   void* out, int B, int Sq, int Hq, int Hkv, int head_dim, int max_kv, int causal,
                                   int window, float scale, rcgqa_dtype dt, void* workspace, size_t workspace_bytes,
                                   rcgqa_stream stream) {
  if (!q || !k_cache || !v_cache || !kv_lens || !out || !good_dtype(dt)) return RCGQA_EINVAL;
  if (!al16({q, k_cache, v_cache, out}) || !al4(kv_lens)) return RCGQA_EINVAL;
  if (out == q || out == k_cache || out == v_cache) return RCGQA_EINVAL;
  if (!pos_int(B) || !pos_int(Sq) || !pos_int(Hq) || !pos_int(Hkv) || Hq % Hkv || !pos_int(max_kv))
    return RCGQA_EINVAL;
  if (head_dim < 2 || head_dim % 2 || (causal != 0 && causal != 1) || !finite_pos(scale)) return RCGQA_EINVAL;
  if (window < 0 || (window > 0 && causal == 0)) return RCGQA_EINVAL;
  if (mul({B, Hq}) > kI32Max || mul({B, Sq, Hq, head_dim}) < 0 || mul({B, Hkv, max_kv, head_dim}) < 0)
    return RCGQA_EINVAL;
  if (!attn_head_dim(head_dim) || !prefill_grid_ok(B, Hq, Sq)) return RCGQA_EUNSUPPORTED;
  if (window >= max_kv) window = 0;  // as attn_prefill_cache: no key is excluded
  const size_t need =
      dt == RCGQA_BF16 ? rcgqa::prefill_cache_split_workspace_bytes(B, Sq, Hq, head_dim, max_kv, causal != 0, window)
                       : 0;
  if (need && (!workspace || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % 256))
    return RCGQA_EINVAL;
  if (workspace && (workspace == q || workspace == k_cache || workspace == v_cache || workspace == out ||
                    workspace == kv_lens))
    return RCGQA_EINVAL;
  const hipStream_t st = (hipStream_t)stream;
  const rcgqa::KvSpec kv{(long long)Hkv * max_kv * head_dim, (long long)max_kv * head_dim, head_dim, kv_lens,
                         max_kv, window};
  if (dt == RCGQA_BF16)
    return hip_status(rcgqa::launch_prefill_bf16_split(q, k_cache, v_cache, out, B, Sq, Hq, Hkv, head_dim,
                                                       causal != 0, scale, kv, need ? workspace : nullptr, st));
  return hip_status(rcgqa::launch_prefill_f32((const float*)q, (const float*)k_cache, (const float*)v_cache,
                                              (float*)out, B, Sq, Hq, Hkv, head_dim, causal != 0, scale, kv, nullptr,
                                              st));
}

rcgqa_status attn_prefill_masked(const void* q, const void* k, const void* v, const void* mask, void* out, int B,
                                 int S, int Hq, int Hkv, int head_dim, int mask_heads, int mask_ld, int causal,
                                 float scale, rcgqa_dtype dt, rcgqa_stream stream) {
  if (!q || !k || !v || !mask || !out || !good_dtype(dt) || !al16({q, k, v, mask, out})) return RCGQA_EINVAL;
  if (out == q || out == k || out == v || out == mask) return RCGQA_EINVAL;
  if (!pos_int(B) || !pos_int(S) || !pos_int(Hq) || !pos_int(Hkv) || Hq % Hkv) return RCGQA_EINVAL;
  if (head_dim < 2 || head_dim % 2 || (causal != 0 && causal != 1) || !finite_pos(scale)) return RCGQA_EINVAL;
  if ((mask_heads != 1 && mask_heads != Hq) || mask_ld < S) return RCGQA_EINVAL;
  if (mul({B, Hq}) > kI32Max || mul({B, S, Hq, head_dim}) < 0 || mul({B, mask_heads, S, mask_ld}) < 0)
    return RCGQA_EINVAL;
  if (!attn_head_dim(head_dim) || !prefill_grid_ok(B, Hq, S)) return RCGQA_EUNSUPPORTED;
  const hipStream_t st = (hipStream_t)stream;
  const long long plane = (long long)S * mask_ld;
  const rcgqa::KvSpec kv{(long long)S * Hkv * head_dim, head_dim, (long long)Hkv * head_dim, nullptr, S, 0,
                         mask, (long long)mask_heads * plane, mask_heads == 1 ? 0 : plane, mask_ld};
  if (dt == RCGQA_BF16)
    return hip_status(
        rcgqa::launch_prefill_bf16(q, k, v, out, B, S, Hq, Hkv, head_dim, causal != 0, scale, kv, nullptr, st));
  return hip_status(rcgqa::launch_prefill_f32((const float*)q, (const float*)k, (const float*)v, (float*)out, B, S,
                                              Hq, Hkv, head_dim, causal != 0, scale, kv, nullptr, st));
}

rcgqa_status attn_prefill_cache(const void* q, const void* k_cache, const void* v_cache, const int32_t* kv_lens,
                                void* out, int B, int Sq, int Hq, int Hkv, int head_dim, int max_kv, int causal,
                                int window, float scale, rcgqa_dtype dt, rcgqa_stream stream) {
  if (!q || !k_cache || !v_cache || !kv_lens || !out || !good_dtype(dt)) return RCGQA_EINVAL;
  if (!al16({q, k_cache, v_cache, out}) || !al4(kv_lens)) return RCGQA_EINVAL;
  if (out == q || out == k_cache || out == v_cache) return RCGQA_EINVAL;
  if (!pos_int(B) || !pos_int(Sq) || !pos_int(Hq) || !pos_int(Hkv) || Hq % Hkv || !pos_int(max_kv))
    return RCGQA_EINVAL;
  if (head_dim < 2 || head_dim % 2 || (causal != 0 && causal != 1) || !finite_pos(scale)) return RCGQA_EINVAL;
  if (window < 0 || (window > 0 && causal == 0)) return RCGQA_EINVAL;
  if (mul({B, Hq}) > kI32Max || mul({B, Sq, Hq, head_dim}) < 0 || mul({B, Hkv, max_kv, head_dim}) < 0)
    return RCGQA_EINVAL;
  if (!attn_head_dim(head_dim) || !prefill_grid_ok(B, Hq, Sq)) return RCGQA_EUNSUPPORTED;
  const hipStream_t st = (hipStream_t)stream;
  // A window of max_kv or more excludes no key (a query sits at a position
  // below max_kv), so it is no window; this also keeps the kernels' position
  // arithmetic (position - window) far from int32 overflow.
  if (window >= max_kv) window = 0;
  // caches [B, Hkv, max_kv, D]: rows of one (batch, KV head) are contiguous
  const rcgqa::KvSpec kv{(long long)Hkv * max_kv * head_dim, (long long)max_kv * head_dim, head_dim, kv_lens,
                         max_kv, window};
  if (dt == RCGQA_BF16)
    return hip_status(rcgqa::launch_prefill_bf16(q, k_cache, v_cache, out, B, Sq, Hq, Hkv, head_dim, causal != 0,
                                                 scale, kv, nullptr, st));
  return hip_status(rcgqa::launch_prefill_f32((const float*)q, (const float*)k_cache, (const float*)v_cache,
                                              (float*)out, B, Sq, Hq, Hkv, head_dim, causal != 0, scale, kv, nullptr,
                                              st));
}

size_t rope_attn_prefill_workspace_bytes(int B, int S, int head_dim) {
  const int64_t n = mul({B, S, head_dim, 4});
  return n < 0 ? 0 : (size_t)n;
}

rcgqa_status rope_attn_prefill(const void* q, void* k, const void* v, void* out, const int32_t* position_ids,
                               int B, int S, int Hq, int Hkv, int head_dim, int causal, float scale, float theta,
                               float linear_factor, rcgqa_dtype dt, void* workspace, size_t workspace_bytes,
                               rcgqa_stream stream) {
  if (!q || !k || !v || !out || !workspace || !good_dtype(dt)) return RCGQA_EINVAL;
  if (!al16({q, k, v, out}) || !al4(position_ids)) return RCGQA_EINVAL;
  if (out == q || out == k || out == v || q == k || k == v) return RCGQA_EINVAL;
  if (!pos_int(B) || !pos_int(S) || !pos_int(Hq) || !pos_int(Hkv) || Hq % Hkv) return RCGQA_EINVAL;
  if (head_dim < 2 || head_dim % 2 || (causal != 0 && causal != 1) || !finite_pos(scale)) return RCGQA_EINVAL;
  if (!finite_pos(theta) || !finite_pos(linear_factor)) return RCGQA_EINVAL;
  const int64_t tokens = mul({B, S});
  if (tokens < 0 || tokens > kI32Max || mul({B, Hq}) > kI32Max || mul({B, S, Hq, head_dim}) < 0) return RCGQA_EINVAL;
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return RCGQA_EINVAL;
  if (!attn_head_dim(head_dim) || !prefill_grid_ok(B, Hq, S)) return RCGQA_EUNSUPPORTED;
  if (workspace_bytes < rope_attn_prefill_workspace_bytes(B, S, head_dim)) return RCGQA_EINVAL;
  const hipStream_t st = (hipStream_t)stream;
  float* table = (float*)workspace;
  // keys rotated in place, each token's cos/sin kept for the queries
  const hipError_t e = rcgqa::launch_rope(nullptr, k, position_ids, B, S, 0, Hkv, head_dim, (double)theta,
                                          (double)linear_factor, dt == RCGQA_BF16, table, st);
  if (e != hipSuccess) return RCGQA_EHIP;
  const rcgqa::KvSpec kv{(long long)S * Hkv * head_dim, head_dim, (long long)Hkv * head_dim, nullptr, S, 0};
  if (dt == RCGQA_BF16)
    return hip_status(
        rcgqa::launch_prefill_bf16(q, k, v, out, B, S, Hq, Hkv, head_dim, causal != 0, scale, kv, table, st));
  return hip_status(rcgqa::launch_prefill_f32((const float*)q, (const float*)k, (const float*)v, (float*)out, B, S,
                                              Hq, Hkv, head_dim, causal != 0, scale, kv, table, st));
}

size_t attn_decode_workspace_bytes(int B, int Hq, int head_dim, int max_kv) {
  if (!pos_int(B) || !pos_int(Hq) || !pos_int(head_dim) || !pos_int(max_kv)) return 0;
  return rcgqa::decode_workspace_bytes(B, Hq, head_dim, max_kv);
}

rcgqa_status attn_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* kv_lens,
                         void* out, int B, int Hq, int Hkv, int head_dim, int max_kv, float scale,
                         rcgqa_dtype dt, void* workspace, size_t workspace_bytes, rcgqa_stream stream) {
  if (!q || !k_cache || !v_cache || !kv_lens || !out || !workspace || !good_dtype(dt)) return RCGQA_EINVAL;
  if (!al16({q, k_cache, v_cache, out}) || !al4(kv_lens)) return RCGQA_EINVAL;
  if (out == q || out == k_cache || out == v_cache) return RCGQA_EINVAL;
  if (!pos_int(B) || !pos_int(Hq) || !pos_int(Hkv) || Hq % Hkv || !pos_int(max_kv)) return RCGQA_EINVAL;
  if (head_dim < 2 || head_dim % 2 || !finite_pos(scale)) return RCGQA_EINVAL;
  if (mul({B, Hkv, max_kv, head_dim}) < 0) return RCGQA_EINVAL;
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return RCGQA_EINVAL;
  if (!attn_head_dim(head_dim) || Hq / Hkv > 16 || B > 65535 || Hq > 65535) return RCGQA_EUNSUPPORTED;
  if (workspace_bytes < rcgqa::decode_workspace_bytes(B, Hq, head_dim, max_kv)) return RCGQA_EINVAL;
  return hip_status(rcgqa::launch_decode(q, k_cache, v_cache, kv_lens, out, B, Hq, Hkv, head_dim, max_kv, scale,
                                         dt == RCGQA_BF16, workspace, (hipStream_t)stream));
}

rcgqa_status attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const int32_t* kv_lens,
                                 void* out, int B, int Hq, int Hkv, int head_dim, int max_kv, float scale,
                                 rcgqa_dtype dt, rcgqa_stream stream) {
  if (!q || !k_cache || !v_cache || !kv_lens || !out || !good_dtype(dt)) return RCGQA_EINVAL;
  if (!al16({q, k_cache, v_cache, out}) || !al4(kv_lens)) return RCGQA_EINVAL;
  if (out == q || out == k_cache || out == v_cache) return RCGQA_EINVAL;
  if (!pos_int(B) || !pos_int(Hq) || !pos_int(Hkv) || Hq % Hkv || !pos_int(max_kv)) return RCGQA_EINVAL;
  if (head_dim < 2 || head_dim % 2 || !finite_pos(scale)) return RCGQA_EINVAL;
  if (mul({B, Hkv, max_kv, head_dim}) < 0) return RCGQA_EINVAL;
  if (!attn_head_dim(head_dim) || Hq / Hkv > 16 || B > 65535 || Hq > 65535) return RCGQA_EUNSUPPORTED;
  const bool bf16 = dt == RCGQA_BF16;
  if (rcgqa::decode_scratch_bytes(B, Hq, head_dim, max_kv, bf16) > rcgqa::kDecodeNoAllocBytes) return RCGQA_ENOSPACE;
  void* ws = nullptr;
  if (rcgqa::decode_noalloc_scratch(&ws) != hipSuccess) return RCGQA_EHIP;
  return hip_status(rcgqa::launch_decode(q, k_cache, v_cache, kv_lens, out, B, Hq, Hkv, head_dim, max_kv, scale,
                                         bf16, ws, (hipStream_t)stream));
}

size_t rope_attn_decode_workspace_bytes(int B, int Hq, int head_dim, int max_kv) {
  if (!pos_int(B) || !pos_int(Hq) || !pos_int(head_dim) || !pos_int(max_kv)) return 0;
  const int64_t qb = mul({B, Hq, head_dim, 4});
  if (qb < 0) return 0;
  return (size_t)((qb + 255) / 256 * 256) + rcgqa::decode_workspace_bytes(B, Hq, head_dim, max_kv);
}

rcgqa_status rope_attn_decode(const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                              const int32_t* kv_lens, const int32_t* position_ids, void* out, int B, int Hq,
                              int Hkv, int head_dim, int max_kv, float scale, float theta, float linear_factor,
                              rcgqa_dtype dt, void* workspace, size_t workspace_bytes, rcgqa_stream stream) {
  if (!q || !k_new || !v_new || !k_cache || !v_cache || !kv_lens || !out || !workspace || !good_dtype(dt))
    return RCGQA_EINVAL;
  if (!al16({q, k_new, v_new, k_cache, v_cache, out}) || !al4(kv_lens) || !al4(position_ids)) return RCGQA_EINVAL;
  if (!pos_int(B) || !pos_int(Hq) || !pos_int(Hkv) || Hq % Hkv || !pos_int(max_kv)) return RCGQA_EINVAL;
  if (head_dim < 2 || head_dim % 2 || !finite_pos(scale)) return RCGQA_EINVAL;
  if (!finite_pos(theta) || !finite_pos(linear_factor)) return RCGQA_EINVAL;
  if (mul({B, Hkv, max_kv, head_dim}) < 0 || mul({B, Hq, head_dim, 4}) < 0) return RCGQA_EINVAL;
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return RCGQA_EINVAL;
  if (!attn_head_dim(head_dim) || Hq / Hkv > 16 || B > 65535 || Hq > 65535) return RCGQA_EUNSUPPORTED;
  if (workspace_bytes < rope_attn_decode_workspace_bytes(B, Hq, head_dim, max_kv)) return RCGQA_EINVAL;
  const hipStream_t st = (hipStream_t)stream;
  // rotated queries first (256-byte aligned), the split-K partial states after them
  const size_t qbytes = ((size_t)B * Hq * head_dim * 4 + 255) / 256 * 256;
  void* q_rot = workspace;
  void* ws = (char*)workspace + qbytes;
  const hipError_t e =
      rcgqa::launch_rope_append(q, q_rot, k_new, v_new, k_cache, v_cache, kv_lens, position_ids, B, Hq, Hkv, head_dim,
                                max_kv, (double)theta, (double)linear_factor, dt == RCGQA_BF16, st);
  if (e != hipSuccess) return RCGQA_EHIP;
  return hip_status(rcgqa::launch_decode(q_rot, k_cache, v_cache, kv_lens, out, B, Hq, Hkv, head_dim, max_kv, scale,
                                         dt == RCGQA_BF16, ws, st));
}

rcgqa_status kv_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new, const int32_t* slots,
                       int B, int Hkv, int head_dim, int max_kv, rcgqa_dtype dt, rcgqa_stream stream) {
  if (!k_cache || !v_cache || !k_new || !v_new || !slots || !good_dtype(dt)) return RCGQA_EINVAL;
  if (!al16({k_cache, v_cache, k_new, v_new}) || !al4(slots)) return RCGQA_EINVAL;
  if (!pos_int(B) || !pos_int(Hkv) || !pos_int(max_kv) || head_dim < 2 || head_dim % 2) return RCGQA_EINVAL;
  if (mul({B, Hkv, max_kv, head_dim}) < 0) return RCGQA_EINVAL;
  if (head_dim > 256 || B > 65535 || Hkv > 65535) return RCGQA_EUNSUPPORTED;
  return hip_status(rcgqa::launch_kv_append(k_cache, v_cache, k_new, v_new, slots, B, Hkv, head_dim, max_kv,
                                            dt == RCGQA_BF16, (hipStream_t)stream));
}

}  // extern "C"
