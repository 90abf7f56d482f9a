// Rotary position embedding, applied in place to Q and K in one pass.
//
// Method: "LLaMA2大语言模型架构详解", section "Rotary Position Encoding" (RoFormer
// rotation of query/key pairs; values untouched), "Llama2 Transformer架构解析与优化实践"
// section 6.1 (linear scaling divides positions by the factor).  Pairing is
// (x[i], x[i + D/2]) with angle (pos / factor) * theta^(-2i/D).
//
// Design: one workgroup per token.  The token's D/2 angles are formed in fp64
// (exact enough for the fp32 path's 1e-5 bound at positions in the thousands)
// and their cos/sin rounded to fp32 into LDS once; every head of q and k at
// that token then reuses them.  Each thread moves 16-byte vectors of the two
// halves of a head vector, so loads and stores are fully coalesced.  The pass
// is HBM-bound: it reads and writes every q/k element once.
#include "common.h"
#include "launch.h"

namespace rcgqa {

template <typename T, int VE>
struct alignas(sizeof(T) * VE) Vec {
  T v[VE];
};

template <typename T, int VE>
__global__ __launch_bounds__(256) void rope_kernel(T* __restrict__ q, T* __restrict__ k,
                                                   const int32_t* __restrict__ pos_ids, int S, int Hq,
                                                   int Hkv, int D, double theta, double factor) {
  extern __shared__ float cs[];  // cos[D/2] then sin[D/2]
  const int tok = blockIdx.x;
  const int half = D >> 1;
  const int pos = pos_ids ? pos_ids[tok] : (tok % S);
  for (int i = threadIdx.x; i < half; i += blockDim.x) {
    const double inv = pow(theta, -2.0 * (double)i / (double)D);
    const double a = ((double)pos / factor) * inv;
    double sn, cn;
    sincos(a, &sn, &cn);
    cs[i] = (float)cn;
    cs[half + i] = (float)sn;
  }
  __syncthreads();
  const int cpr = half / VE;  // vectors per half head-vector
  const int units = (Hq + Hkv) * cpr;
  for (int u = threadIdx.x; u < units; u += blockDim.x) {
    const int head = u / cpr, c = u - head * cpr;
    T* base = head < Hq ? q + ((size_t)tok * Hq + head) * D : k + ((size_t)tok * Hkv + (head - Hq)) * D;
    Vec<T, VE>* p1 = reinterpret_cast<Vec<T, VE>*>(base + c * VE);
    Vec<T, VE>* p2 = reinterpret_cast<Vec<T, VE>*>(base + half + c * VE);
    Vec<T, VE> x1 = *p1, x2 = *p2, y1, y2;
#pragma unroll
    for (int e = 0; e < VE; e++) {
      const float co = cs[c * VE + e], si = cs[half + c * VE + e];
      const float a = (float)x1.v[e], b = (float)x2.v[e];
      y1.v[e] = (T)fmaf(a, co, -(b * si));
      y2.v[e] = (T)fmaf(b, co, a * si);
    }
    *p1 = y1;
    *p2 = y2;
  }
}

hipError_t launch_rope(void* q, void* k, const int32_t* pos, int B, int S, int Hq, int Hkv, int D,
                       double theta, double factor, bool bf16_io, hipStream_t st) {
  const dim3 grid((unsigned)((long)B * S)), block(256);
  const size_t lds = (size_t)D * sizeof(float);
  const int half = D / 2;
  if (bf16_io) {
    if (half % 8 == 0)
      hipLaunchKernelGGL((rope_kernel<bf16, 8>), grid, block, lds, st, (bf16*)q, (bf16*)k, pos, S, Hq, Hkv, D,
                         theta, factor);
    else
      hipLaunchKernelGGL((rope_kernel<bf16, 1>), grid, block, lds, st, (bf16*)q, (bf16*)k, pos, S, Hq, Hkv, D,
                         theta, factor);
  } else {
    if (half % 4 == 0)
      hipLaunchKernelGGL((rope_kernel<float, 4>), grid, block, lds, st, (float*)q, (float*)k, pos, S, Hq, Hkv,
                         D, theta, factor);
    else
      hipLaunchKernelGGL((rope_kernel<float, 1>), grid, block, lds, st, (float*)q, (float*)k, pos, S, Hq, Hkv,
                         D, theta, factor);
  }
  return hipGetLastError();
}

}  // namespace rcgqa
