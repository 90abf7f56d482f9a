// Rotary position embedding, applied in place to Q and K in one pass.
//
// Method: "LLaMA2大语言模型架构详解", section "Rotary Position Encoding" (RoFormer
// rotation of query/key pairs; values untouched), "Llama2 Transformer架构解析与优化实践"
// section 6.1 (linear scaling divides positions by the factor).  Pairing is
// (x[i], x[i + D/2]) with angle (pos / factor) * theta^(-2i/D).
//
// Design: one workgroup per token (a workgroup takes several tokens, a grid
// apart, only when there are more than kMaxTokenGroups).  The token's D/2 angles are formed in fp64
// (exact enough for the fp32 path's 1e-5 bound at positions in the thousands)
// and their cos/sin rounded to fp32 into LDS once; every head of q and k at
// that token then reuses them.  Each thread moves 16-byte vectors of the two
// halves of a head vector, so loads and stores are fully coalesced.  The pass
// is HBM-bound: it reads and writes every q/k element once.
//
// The interleaved pairing (x[2i], x[2i+1]) -- the complex-pair form of the
// same rotation -- has its own kernel: each 16-byte vector then holds whole
// pairs, with the same angles and arithmetic per pair.
//
// For the fused paths the same kernel can rotate K alone and write the
// token's cos/sin row to a table (the prefill kernel then rotates Q as it
// loads it, with the very same values and arithmetic), and a second kernel
// rotates a decode step's q and new key and appends the key and value to the
// cache in one launch.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace rcgqa {

// Largest grid of the per-token kernels: 2^20 workgroups of 256 work-items
// keep the launch far inside the 32-bit work-item count of a dispatch.
constexpr int kMaxTokenGroups = 1 << 20;
constexpr int kMinTokenGroups = 2048;

template <typename T, int VE>
struct alignas(sizeof(T) * VE) Vec {
  T v[VE];
};

__device__ __forceinline__ void rope_angles(float* cs, int pos, int D, double theta, double factor) {
  const int half = D >> 1;
  for (int i = threadIdx.x; i < half; i += blockDim.x) {
    const double inv = pow(theta, -2.0 * (double)i / (double)D);
    const double a = ((double)pos / factor) * inv;
    double sn, cn;
    sincos(a, &sn, &cn);
    cs[i] = (float)cn;
    cs[half + i] = (float)sn;
  }
}

// (x1, x2) -> (x1 c - x2 s, x2 c + x1 s) in fp32, rounded once to T: VE
// elements of each half of one head vector, read at s1/s2 and written to d1/d2
// (which may be the same addresses).
template <typename T, int VE>
__device__ __forceinline__ void rope_pair(const T* s1, const T* s2, T* d1, T* d2, const float* cs, int c, int half) {
  const Vec<T, VE> x1 = *reinterpret_cast<const Vec<T, VE>*>(s1), x2 = *reinterpret_cast<const Vec<T, VE>*>(s2);
  Vec<T, VE> y1, y2;
#pragma unroll
  for (int e = 0; e < VE; e++) {
    const float co = cs[c * VE + e], si = cs[half + c * VE + e];
    const float a = (float)x1.v[e], b = (float)x2.v[e];
    y1.v[e] = (T)fmaf(a, co, -(b * si));
    y2.v[e] = (T)fmaf(b, co, a * si);
  }
  *reinterpret_cast<Vec<T, VE>*>(d1) = y1;
  *reinterpret_cast<Vec<T, VE>*>(d2) = y2;
}

// q may be null with Hq == 0 (keys only); table, when not null, receives the
// token's cos/sin row: table[tok * D + i] = cos, table[tok * D + D/2 + i] = sin.
// A workgroup takes tpi consecutive tokens at a time (tpi * D/2 <= 256 when
// tpi > 1): the inverse frequencies are formed once per workgroup, the tpi
// tokens' angles are spread over its threads, then their q/k vectors are
// rotated.  The angles and arithmetic do not depend on tpi.
template <typename T, int VE>
__global__ __launch_bounds__(256) void rope_kernel(T* __restrict__ q, T* __restrict__ k,
                                                   const int32_t* __restrict__ pos_ids, long long ntok, int S,
                                                   int Hq, int Hkv, int D, double theta, double factor,
                                                   float* __restrict__ table, int tpi) {
  extern __shared__ float cs[];  // tpi rows of cos[D/2] then sin[D/2], then the inverse frequencies (double)
  const int half = D >> 1;
  double* const inv = reinterpret_cast<double*>(cs + (size_t)tpi * D);
  for (int i = threadIdx.x; i < half; i += blockDim.x) inv[i] = pow(theta, -2.0 * (double)i / (double)D);
  const int cpr = half / VE;  // vectors per half head-vector
  const int units = (Hq + Hkv) * cpr;
  for (long long t0 = (long long)blockIdx.x * tpi; t0 < ntok; t0 += (long long)gridDim.x * tpi) {
    __syncthreads();  // inv written / the previous tokens' cs fully read
    const int nt = ntok - t0 < tpi ? (int)(ntok - t0) : tpi;
    for (int j = threadIdx.x; j < nt * half; j += blockDim.x) {
      const int tt = j / half, i = j - tt * half;
      const long long tok = t0 + tt;
      const int pos = pos_ids ? pos_ids[tok] : (int)(tok % S);
      const double a = ((double)pos / factor) * inv[i];
      double sn, cn;
      sincos(a, &sn, &cn);
      cs[tt * D + i] = (float)cn;
      cs[tt * D + half + i] = (float)sn;
    }
    __syncthreads();
    if (table)
      for (int j = threadIdx.x; j < nt * D; j += blockDim.x) table[(size_t)t0 * D + j] = cs[j];
    for (int u = threadIdx.x; u < nt * units; u += blockDim.x) {
      const int tt = u / units, r = u - tt * units;
      const int head = r / cpr, c = r - head * cpr;
      const long long tok = t0 + tt;
      T* base = head < Hq ? q + ((size_t)tok * Hq + head) * D : k + ((size_t)tok * Hkv + (head - Hq)) * D;
      rope_pair<T, VE>(base + c * VE, base + half + c * VE, base + c * VE, base + half + c * VE, cs + tt * D, c, half);
    }
  }
}

// Interleaved pairs: VE elements (VE/2 whole pairs) per vector, pair i of a
// head vector is (x[2i], x[2i+1]) with the angle of frequency index i.
template <typename T, int VE>
__global__ __launch_bounds__(256) void rope_interleaved_kernel(T* __restrict__ q, T* __restrict__ k,
                                                               const int32_t* __restrict__ pos_ids,
                                                               long long ntok, int S, int Hq, int Hkv, int D,
                                                               double theta, double factor) {
  extern __shared__ float cs[];  // cos[D/2] then sin[D/2]
  const int half = D >> 1;
  const int cpr = D / VE;  // vectors per head vector
  const int units = (Hq + Hkv) * cpr;
  for (long long tok = blockIdx.x; tok < ntok; tok += gridDim.x) {
    if (tok != (long long)blockIdx.x) __syncthreads();  // the previous token's cs fully read
    const int pos = pos_ids ? pos_ids[tok] : (int)(tok % S);
    rope_angles(cs, pos, D, theta, factor);
    __syncthreads();
    for (int u = threadIdx.x; u < units; u += blockDim.x) {
      const int head = u / cpr, c = u - head * cpr;
      T* p = (head < Hq ? q + ((size_t)tok * Hq + head) * D : k + ((size_t)tok * Hkv + (head - Hq)) * D) + c * VE;
      const Vec<T, VE> x = *reinterpret_cast<const Vec<T, VE>*>(p);
      Vec<T, VE> y;
#pragma unroll
      for (int j = 0; j < VE / 2; j++) {
        const int i = c * (VE / 2) + j;
        const float co = cs[i], si = cs[half + i];
        const float a = (float)x.v[2 * j], b = (float)x.v[2 * j + 1];
        y.v[2 * j] = (T)fmaf(a, co, -(b * si));
        y.v[2 * j + 1] = (T)fmaf(b, co, a * si);
      }
      *reinterpret_cast<Vec<T, VE>*>(p) = y;
    }
  }
}

// One decode step per sequence b (one workgroup each): rotate q[b] into
// q_out[b] and k_new[b] at position pos_b, then write the rotated key and
// v_new[b] into cache row slot_b = kv_lens[b] - 1 (nothing is written when
// that row is outside [0, max_kv)).  pos_b = pos_ids[b], or slot_b when
// pos_ids is null.  Same angles and arithmetic as rope_kernel.
template <typename T, int VE>
__global__ __launch_bounds__(256) void rope_append_kernel(const T* __restrict__ q, T* __restrict__ q_out,
                                                          const T* __restrict__ k_new, const T* __restrict__ v_new,
                                                          T* __restrict__ k_cache, T* __restrict__ v_cache,
                                                          const int32_t* __restrict__ kv_lens,
                                                          const int32_t* __restrict__ pos_ids, int Hq, int Hkv,
                                                          int D, int max_kv, double theta, double factor) {
  extern __shared__ float cs[];
  const int b = blockIdx.x;
  const int half = D >> 1;
  const int len = kv_lens[b];
  const int slot = len > 0 ? len - 1 : -1;  // no overflow for any int32 length
  const int pos = pos_ids ? pos_ids[b] : slot;
  const bool write = slot >= 0 && slot < max_kv;
  rope_angles(cs, pos, D, theta, factor);
  __syncthreads();
  const int cpr = half / VE;
  for (int u = threadIdx.x; u < Hq * cpr; u += blockDim.x) {
    const int head = u / cpr, c = u - head * cpr;
    const size_t off = ((size_t)b * Hq + head) * D;
    rope_pair<T, VE>(q + off + c * VE, q + off + half + c * VE, q_out + off + c * VE, q_out + off + half + c * VE, cs,
                     c, half);
  }
  if (!write) return;
  for (int u = threadIdx.x; u < Hkv * cpr; u += blockDim.x) {
    const int head = u / cpr, c = u - head * cpr;
    const size_t src = ((size_t)b * Hkv + head) * D;
    const size_t dst = (((size_t)b * Hkv + head) * max_kv + slot) * D;
    rope_pair<T, VE>(k_new + src + c * VE, k_new + src + half + c * VE, k_cache + dst + c * VE,
                     k_cache + dst + half + c * VE, cs, c, half);
    *reinterpret_cast<Vec<T, VE>*>(v_cache + dst + c * VE) = *reinterpret_cast<const Vec<T, VE>*>(v_new + src + c * VE);
    *reinterpret_cast<Vec<T, VE>*>(v_cache + dst + half + c * VE) =
        *reinterpret_cast<const Vec<T, VE>*>(v_new + src + half + c * VE);
  }
}

hipError_t launch_rope(void* q, void* k, const int32_t* pos, int B, int S, int Hq, int Hkv, int D,
                       double theta, double factor, bool bf16_io, float* table, hipStream_t st) {
  const long long ntok = (long long)B * S;
  const int half = D / 2;
  // Several tokens per workgroup only while the grid keeps at least
  // kMinTokenGroups workgroups (8 per CU); short launches keep one token each.
  const long long fill = ntok / kMinTokenGroups;
  const int tpi = (int)std::max(1LL, std::min(fill, (long long)(half <= 256 ? 256 / half : 1)));
  const long long groups = (ntok + tpi - 1) / tpi;
  const dim3 grid((unsigned)(groups < kMaxTokenGroups ? groups : kMaxTokenGroups)), block(256);
  const size_t lds = (size_t)tpi * D * sizeof(float) + (size_t)half * sizeof(double);
  if (bf16_io) {
    if (half % 8 == 0)
      hipLaunchKernelGGL((rope_kernel<bf16, 8>), grid, block, lds, st, (bf16*)q, (bf16*)k, pos, ntok, S, Hq, Hkv, D,
                         theta, factor, table, tpi);
    else
      hipLaunchKernelGGL((rope_kernel<bf16, 1>), grid, block, lds, st, (bf16*)q, (bf16*)k, pos, ntok, S, Hq, Hkv, D,
                         theta, factor, table, tpi);
  } else {
    if (half % 4 == 0)
      hipLaunchKernelGGL((rope_kernel<float, 4>), grid, block, lds, st, (float*)q, (float*)k, pos, ntok, S, Hq, Hkv,
                         D, theta, factor, table, tpi);
    else
      hipLaunchKernelGGL((rope_kernel<float, 1>), grid, block, lds, st, (float*)q, (float*)k, pos, ntok, S, Hq, Hkv,
                         D, theta, factor, table, tpi);
  }
  return hipGetLastError();
}

hipError_t launch_rope_interleaved(void* q, void* k, const int32_t* pos, int B, int S, int Hq, int Hkv, int D,
                                  double theta, double factor, bool bf16_io, hipStream_t st) {
  const long long ntok = (long long)B * S;
  const dim3 grid((unsigned)(ntok < kMaxTokenGroups ? ntok : kMaxTokenGroups)), block(256);
  const size_t lds = (size_t)D * sizeof(float);
  if (bf16_io) {
    if (D % 8 == 0)
      hipLaunchKernelGGL((rope_interleaved_kernel<bf16, 8>), grid, block, lds, st, (bf16*)q, (bf16*)k, pos, ntok, S, Hq,
                         Hkv, D, theta, factor);
    else
      hipLaunchKernelGGL((rope_interleaved_kernel<bf16, 2>), grid, block, lds, st, (bf16*)q, (bf16*)k, pos, ntok, S, Hq,
                         Hkv, D, theta, factor);
  } else {
    if (D % 4 == 0)
      hipLaunchKernelGGL((rope_interleaved_kernel<float, 4>), grid, block, lds, st, (float*)q, (float*)k, pos, ntok, S,
                         Hq, Hkv, D, theta, factor);
    else
      hipLaunchKernelGGL((rope_interleaved_kernel<float, 2>), grid, block, lds, st, (float*)q, (float*)k, pos, ntok, S,
                         Hq, Hkv, D, theta, factor);
  }
  return hipGetLastError();
}

hipError_t launch_rope_append(const void* q, void* q_out, const void* k_new, const void* v_new, void* k_cache,
                              void* v_cache, const int32_t* kv_lens, const int32_t* pos, int B, int Hq, int Hkv,
                              int D, int max_kv, double theta, double factor, bool bf16_io, hipStream_t st) {
  const dim3 grid((unsigned)B), block(256);
  const size_t lds = (size_t)D * sizeof(float);
  const int half = D / 2;
  if (bf16_io) {
    if (half % 8 == 0)
      hipLaunchKernelGGL((rope_append_kernel<bf16, 8>), grid, block, lds, st, (const bf16*)q, (bf16*)q_out,
                         (const bf16*)k_new, (const bf16*)v_new, (bf16*)k_cache, (bf16*)v_cache, kv_lens, pos, Hq,
                         Hkv, D, max_kv, theta, factor);
    else
      hipLaunchKernelGGL((rope_append_kernel<bf16, 1>), grid, block, lds, st, (const bf16*)q, (bf16*)q_out,
                         (const bf16*)k_new, (const bf16*)v_new, (bf16*)k_cache, (bf16*)v_cache, kv_lens, pos, Hq,
                         Hkv, D, max_kv, theta, factor);
  } else {
    if (half % 4 == 0)
      hipLaunchKernelGGL((rope_append_kernel<float, 4>), grid, block, lds, st, (const float*)q, (float*)q_out,
                         (const float*)k_new, (const float*)v_new, (float*)k_cache, (float*)v_cache, kv_lens, pos,
                         Hq, Hkv, D, max_kv, theta, factor);
    else
      hipLaunchKernelGGL((rope_append_kernel<float, 1>), grid, block, lds, st, (const float*)q, (float*)q_out,
                         (const float*)k_new, (const float*)v_new, (float*)k_cache, (float*)v_cache, kv_lens, pos,
                         Hq, Hkv, D, max_kv, theta, factor);
  }
  return hipGetLastError();
}

}  // namespace rcgqa
