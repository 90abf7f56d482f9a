// fp32 prefill attention: exact fp32 arithmetic for the fp32 path.
//
// Method: "【HuggingFace Transformers】LlamaAttention源码解析", section 1.2 steps 2-4
// (scaled scores, additive causal mask, softmax, weights @ V); query head h
// reads K/V head h / G (repeat_kv, section 2 step 4).
//
// Design: one wave per 64 query rows of one (batch, head); each lane owns one
// query row (q and the fp32 accumulator in registers) and walks the keys with
// an online softmax using the accurate expf.  K/V tiles of 32 keys are staged
// in LDS and read as wave-wide broadcasts.  Causal tiles past the block's last
// row are never loaded.  This path targets accuracy (1e-5 against fp64), not
// throughput.
#include "common.h"
#include "launch.h"

namespace rcgqa {

template <int D>
__global__ __launch_bounds__(64) void prefill_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                         const float* __restrict__ v, float* __restrict__ out,
                                                         int S, int Hq, int Hkv, int causal, float scale) {
  constexpr int BM = 64, BN = 32;
  __shared__ float4 sk[BN * D / 4], sv[BN * D / 4];
  const int bh = blockIdx.x, b = bh / Hq, h = bh - b * Hq;
  const int kvh = h / (Hq / Hkv);
  const int q0 = blockIdx.y * BM, i = q0 + threadIdx.x;
  const bool live = i < S;
  const size_t qrs = (size_t)Hq * D, kvrs = (size_t)Hkv * D;
  const float* kb = k + (size_t)b * S * kvrs + (size_t)kvh * D;
  const float* vb = v + (size_t)b * S * kvrs + (size_t)kvh * D;

  float qr[D], acc[D];
  const float* qp = q + ((size_t)b * S + (live ? i : 0)) * qrs + (size_t)h * D;
#pragma unroll
  for (int d = 0; d < D; d++) {
    qr[d] = live ? qp[d] : 0.f;
    acc[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int kv_end = causal ? min(S, q0 + BM) : S;
  for (int kv0 = 0; kv0 < kv_end; kv0 += BN) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < BN * D / 4; idx += 64) {
      const int r = idx / (D / 4), c = idx - r * (D / 4), key = kv0 + r;
      float4 kk = {0.f, 0.f, 0.f, 0.f}, vv = kk;
      if (key < S) {
        kk = reinterpret_cast<const float4*>(kb + (size_t)key * kvrs)[c];
        vv = reinterpret_cast<const float4*>(vb + (size_t)key * kvrs)[c];
      }
      sk[idx] = kk;
      sv[idx] = vv;
    }
    __syncthreads();
    if (!live) continue;
    const int jn = min(BN, S - kv0);
    for (int j = 0; j < jn; j++) {
      const int key = kv0 + j;
      if (causal && key > i) break;
      const float* kr = reinterpret_cast<const float*>(sk) + j * D;
      const float* vr = reinterpret_cast<const float*>(sv) + j * D;
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < D; d++) dot = fmaf(qr[d], kr[d], dot);
      const float s = dot * scale;
      if (s > m) {
        const float corr = expf(m - s);
        l *= corr;
#pragma unroll
        for (int d = 0; d < D; d++) acc[d] *= corr;
        m = s;
      }
      const float p = expf(s - m);
      l += p;
#pragma unroll
      for (int d = 0; d < D; d++) acc[d] = fmaf(p, vr[d], acc[d]);
    }
  }
  if (!live) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float* op = out + ((size_t)b * S + i) * qrs + (size_t)h * D;
#pragma unroll
  for (int d = 0; d < D; d++) op[d] = acc[d] * inv;
}

hipError_t launch_prefill_f32(const float* q, const float* k, const float* v, float* out, int B, int S, int Hq,
                              int Hkv, int D, bool causal, float scale, hipStream_t st) {
  const dim3 grid((unsigned)(B * Hq), (unsigned)((S + 63) / 64)), block(64);
  if (D == 64)
    hipLaunchKernelGGL(prefill_f32_kernel<64>, grid, block, 0, st, q, k, v, out, S, Hq, Hkv, (int)causal, scale);
  else
    hipLaunchKernelGGL(prefill_f32_kernel<128>, grid, block, 0, st, q, k, v, out, S, Hq, Hkv, (int)causal, scale);
  return hipGetLastError();
}

}  // namespace rcgqa
