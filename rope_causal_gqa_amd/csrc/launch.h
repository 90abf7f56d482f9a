// Internal launchers (host side) of librcgqa; arguments are validated by the
// C-ABI layer before any of these is called.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rcgqa {

hipError_t launch_rope(void* q, void* k, const int32_t* pos, int B, int S, int Hq, int Hkv, int D,
                       double theta, double factor, bool bf16, hipStream_t st);

hipError_t launch_prefill_f32(const float* q, const float* k, const float* v, float* out, int B, int S,
                              int Hq, int Hkv, int D, bool causal, float scale, hipStream_t st);

hipError_t launch_prefill_bf16(const void* q, const void* k, const void* v, void* out, int B, int S,
                               int Hq, int Hkv, int D, bool causal, float scale, hipStream_t st);

// Split-K decode: partial softmax states go to `ws`, then a merge pass writes out.
size_t decode_workspace_bytes(int B, int Hq, int D, int max_kv);
hipError_t launch_decode(const void* q, const void* kc, const void* vc, const int32_t* kv_lens, void* out,
                         int B, int Hq, int Hkv, int D, int max_kv, float scale, bool bf16, void* ws,
                         hipStream_t st);

hipError_t launch_kv_append(void* kc, void* vc, const void* kn, const void* vn, const int32_t* slots, int B,
                            int Hkv, int D, int max_kv, bool bf16, hipStream_t st);

}  // namespace rcgqa
