// Single-token decode against a KV cache, split over the key axis.
//
// Method: "LLaMA2大语言模型架构详解", section "KV cache" (the new token's query
// scores every cached key; earlier rows are not recomputed) and section
// "Grouped Multi-Query Attention" (G query heads share one K/V stream);
// softmax as in "【HuggingFace Transformers】LlamaAttention源码解析" section 1.2.
//
// The sequence of one (batch, KV head) is cut into chunks of KC keys.  Pass 1
// writes, per (batch, query head, chunk), the chunk's running max m, sum l and
// unnormalised accumulator acc[D] (all fp32) to the workspace.  Pass 2 merges
// the chunks of a row in a fixed order:
//     M = max_c m_c,  out = sum_c e^(m_c - M) acc_c / sum_c e^(m_c - M) l_c.
// The split is what lets short and long sequences share the GPU evenly; the
// fixed merge order keeps results bitwise repeatable.
#include "common.h"
#include "launch.h"

namespace rcgqa {

namespace {
constexpr int KC = 256;  // keys per chunk (and threads per pass-1 workgroup)
}

size_t decode_workspace_bytes(int B, int Hq, int D, int max_kv) {
  const size_t nch = ((size_t)max_kv + KC - 1) / KC;
  return (size_t)B * Hq * nch * (size_t)(D + 2) * sizeof(float);
}

template <typename T>
__device__ __forceinline__ float to_f(T x) { return (float)x; }

// Pass 1, simple form: one workgroup per (chunk, query head, batch); thread t
// scores key c0 + t, then threads d < D accumulate column d of P V.
template <typename T, int D>
__global__ __launch_bounds__(KC) void decode_chunk_kernel(const T* __restrict__ q, const T* __restrict__ kc,
                                                          const T* __restrict__ vc,
                                                          const int32_t* __restrict__ kv_lens,
                                                          float* __restrict__ ws, int Hq, int Hkv, int max_kv,
                                                          float scale) {
  __shared__ float qs[D];
  __shared__ float ps[KC];
  __shared__ float red[KC / 64];
  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int nch = (int)gridDim.x;
  const int L = min(max(kv_lens[b], 0), max_kv);
  const int c0 = chunk * KC;
  if (c0 >= L) return;  // uniform: this chunk holds no valid key
  const int kvh = h / (Hq / Hkv);
  const size_t head_base = ((size_t)b * Hkv + kvh) * (size_t)max_kv * D;
  for (int d = t; d < D; d += KC) qs[d] = to_f(q[((size_t)b * Hq + h) * D + d]);
  __syncthreads();

  const int key = c0 + t;
  const bool valid = key < L;
  float s = -INFINITY;
  if (valid) {
    const T* kr = kc + head_base + (size_t)key * D;
    float dot = 0.f;
#pragma unroll 8
    for (int d = 0; d < D; d++) dot = fmaf(qs[d], to_f(kr[d]), dot);
    s = dot * scale;
  }
  // workgroup max
  float mx = s;
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if ((t & 63) == 0) red[t >> 6] = mx;
  __syncthreads();
  mx = red[0];
#pragma unroll
  for (int i = 1; i < KC / 64; i++) mx = fmaxf(mx, red[i]);
  __syncthreads();
  const float p = valid ? expf(s - mx) : 0.f;
  ps[t] = p;
  float sm = p;
  for (int o = 32; o > 0; o >>= 1) sm += __shfl_xor(sm, o);
  if ((t & 63) == 0) red[t >> 6] = sm;
  __syncthreads();
  float l = 0.f;
#pragma unroll
  for (int i = 0; i < KC / 64; i++) l += red[i];

  float* dst = ws + (((size_t)b * Hq + h) * nch + chunk) * (D + 2);
  const int jn = min(KC, L - c0);
  for (int d = t; d < D; d += KC) {
    float acc = 0.f;
    const T* vr = vc + head_base + (size_t)c0 * D + d;
    for (int j = 0; j < jn; j++) acc = fmaf(ps[j], to_f(vr[(size_t)j * D]), acc);
    dst[2 + d] = acc;
  }
  if (t == 0) {
    dst[0] = mx;
    dst[1] = l;
  }
}

// Pass 2: one workgroup per (query head, batch), thread d owns output column d.
template <typename T, int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(const float* __restrict__ ws,
                                                         const int32_t* __restrict__ kv_lens, T* __restrict__ out,
                                                         int Hq, int max_kv, int nch) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int L = min(max(kv_lens[b], 0), max_kv);
  const int n = (L + KC - 1) / KC;
  const float* src = ws + ((size_t)b * Hq + h) * nch * (D + 2);
  float M = -INFINITY;
  for (int c = 0; c < n; c++) M = fmaxf(M, src[c * (D + 2)]);
  float num = 0.f, den = 0.f;
  for (int c = 0; c < n; c++) {
    const float e = expf(src[c * (D + 2)] - M);
    den = fmaf(e, src[c * (D + 2) + 1], den);
    num = fmaf(e, src[c * (D + 2) + 2 + d], num);
  }
  out[((size_t)b * Hq + h) * D + d] = (T)(n > 0 ? num / den : 0.f);
}

template <typename T, int D>
static void launch_decode_t(const void* q, const void* kc, const void* vc, const int32_t* kv_lens, void* out, int B,
                            int Hq, int Hkv, int max_kv, float scale, void* ws, hipStream_t st) {
  const int nch = (max_kv + KC - 1) / KC;
  hipLaunchKernelGGL((decode_chunk_kernel<T, D>), dim3(nch, Hq, B), dim3(KC), 0, st, (const T*)q, (const T*)kc,
                     (const T*)vc, kv_lens, (float*)ws, Hq, Hkv, max_kv, scale);
  hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3(Hq, B), dim3(D), 0, st, (const float*)ws, kv_lens, (T*)out,
                     Hq, max_kv, nch);
}

hipError_t launch_decode(const void* q, const void* kc, const void* vc, const int32_t* kv_lens, void* out, int B,
                         int Hq, int Hkv, int D, int max_kv, float scale, bool bf16_io, void* ws, hipStream_t st) {
  if (bf16_io) {
    if (D == 64) launch_decode_t<bf16, 64>(q, kc, vc, kv_lens, out, B, Hq, Hkv, max_kv, scale, ws, st);
    else launch_decode_t<bf16, 128>(q, kc, vc, kv_lens, out, B, Hq, Hkv, max_kv, scale, ws, st);
  } else {
    if (D == 64) launch_decode_t<float, 64>(q, kc, vc, kv_lens, out, B, Hq, Hkv, max_kv, scale, ws, st);
    else launch_decode_t<float, 128>(q, kc, vc, kv_lens, out, B, Hq, Hkv, max_kv, scale, ws, st);
  }
  return hipGetLastError();
}

// Cache append: block (b, kv head) copies one row of k_new and v_new into
// row slots[b] of the caches.
template <typename T>
__global__ void kv_append_kernel(T* __restrict__ kc, T* __restrict__ vc, const T* __restrict__ kn,
                                 const T* __restrict__ vn, const int32_t* __restrict__ slots, int Hkv, int D,
                                 int max_kv) {
  const int b = blockIdx.y, h = blockIdx.x;
  const int s = slots[b];
  if (s < 0 || s >= max_kv) return;
  const size_t dst = (((size_t)b * Hkv + h) * max_kv + s) * D, src = ((size_t)b * Hkv + h) * D;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    kc[dst + d] = kn[src + d];
    vc[dst + d] = vn[src + d];
  }
}

hipError_t launch_kv_append(void* kc, void* vc, const void* kn, const void* vn, const int32_t* slots, int B,
                            int Hkv, int D, int max_kv, bool bf16_io, hipStream_t st) {
  const dim3 grid(Hkv, B), block(64);
  if (bf16_io)
    hipLaunchKernelGGL(kv_append_kernel<bf16>, grid, block, 0, st, (bf16*)kc, (bf16*)vc, (const bf16*)kn,
                       (const bf16*)vn, slots, Hkv, D, max_kv);
  else
    hipLaunchKernelGGL(kv_append_kernel<float>, grid, block, 0, st, (float*)kc, (float*)vc, (const float*)kn,
                       (const float*)vn, slots, Hkv, D, max_kv);
  return hipGetLastError();
}

}  // namespace rcgqa
