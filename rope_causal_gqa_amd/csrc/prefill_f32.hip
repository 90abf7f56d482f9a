// fp32 prefill attention: exact fp32 arithmetic for the fp32 path.
//
// Method: "【HuggingFace Transformers】LlamaAttention源码解析", section 1.2 steps 2-4
// (scaled scores, additive causal mask, softmax, weights @ V); query head h
// reads K/V head h / G (repeat_kv, section 2 step 4).
//
// Design: one workgroup of four waves per 64 query rows of one (batch, head).
// Each lane owns one query row (q and an fp32 accumulator in registers); the
// four waves take the same rows and every fourth key of each 32-key K/V tile,
// each with its own online softmax (accurate expf), and their states are
// merged in a fixed order at the end.  The tiles are staged in LDS and read
// as wave-wide broadcasts, a whole K or V row per batch of reads; dot
// products run as four partial sums.  (A lone wave hides no latency by
// itself: without these, each LDS read and each FMA of a chain was waited
// out.)  Causal tiles past the block's last
// row (and, with a sliding window, before its first window) are never loaded.
// Keys come through strides and per-sequence counts, so the same kernel serves
// chunked / variable-length prefill against a cache; an optional additive
// mask (plain layout) is added to each scaled score.  Given a per-token
// cos/sin table, each lane first rotates its query row (RoPE fused into the
// load, same arithmetic as the RoPE kernel).  This path targets accuracy
// (1e-5 against fp64), not throughput.
#include "common.h"
#include "launch.h"

namespace rcgqa {

constexpr int kF32Waves = 4;  // waves per workgroup, splitting each tile's keys

template <int D>
__global__ __launch_bounds__(64 * kF32Waves) void prefill_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                         const float* __restrict__ v, float* __restrict__ out,
                                                         int Sq, int Hq, int Hkv, int causal, float scale,
                                                         KvSpec kv, const float* __restrict__ q_rope) {
  constexpr int BM = 64, BN = 32, NWV = kF32Waves;
  constexpr int TILE4 = BN * D / 4;                 // float4 per K (or V) tile
  constexpr int MERGE = (NWV - 1) * (D + 2) * 64;   // floats: states of waves 1.. for the merge
  constexpr int SH4 = 2 * TILE4 > MERGE / 4 ? 2 * TILE4 : MERGE / 4;
  __shared__ float4 sh[SH4];  // the K and V tiles, then the merge area
  float4* const sk = sh;
  float4* const sv = sh + TILE4;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int bh = blockIdx.x, b = bh / Hq, h = bh - b * Hq;
  const int kvh = h / (Hq / Hkv);
  const int q0 = blockIdx.y * BM, i = q0 + lane;
  const bool live = i < Sq;
  const size_t qrs = (size_t)Hq * D, kvrs = (size_t)kv.sr;
  const float* kb = k + (size_t)b * kv.sb + (size_t)kvh * kv.sh;
  const float* vb = v + (size_t)b * kv.sb + (size_t)kvh * kv.sh;
  // this sequence's keys; query i sits at absolute position i + off
  const int nk = kv.lens ? min(max(kv.lens[b], 0), kv.max_kv) : Sq;
  const int off = nk - Sq, W = kv.window;
  const int pos = i + off;

  float qr[D], acc[D];
  const float* qp = q + ((size_t)b * Sq + (live ? i : 0)) * qrs + (size_t)h * D;
#pragma unroll
  for (int d = 0; d < D; d++) {
    qr[d] = live ? qp[d] : 0.f;
    acc[d] = 0.f;
  }
  if (q_rope && live) {  // rotate the query row by its token's cos/sin (same arithmetic as rope_apply)
    const float* cs = q_rope + ((size_t)b * Sq + i) * D;
#pragma unroll
    for (int d = 0; d < D / 2; d++) {
      const float co = cs[d], si = cs[D / 2 + d], a = qr[d], bb = qr[D / 2 + d];
      qr[d] = fmaf(a, co, -(bb * si));
      qr[D / 2 + d] = fmaf(bb, co, a * si);
    }
  }
  const float* mrow = kv.mask && live ? reinterpret_cast<const float*>(kv.mask) + (size_t)b * kv.msb +
                                            (size_t)h * kv.msh + (size_t)i * kv.msr
                                      : nullptr;
  float m = -INFINITY, l = 0.f;
  // keys any row of this block can see: [key_lo, key_hi)
  const int key_hi = causal ? min(nk, q0 + BM + off) : nk;
  const int key_lo = (causal && W > 0) ? max(0, q0 + off - W + 1) / BN * BN : 0;
  for (int kv0 = key_lo; kv0 < key_hi; kv0 += BN) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < TILE4; idx += 64 * NWV) {
      const int r = idx / (D / 4), c = idx - r * (D / 4), key = kv0 + r;
      float4 kk = {0.f, 0.f, 0.f, 0.f}, vv = kk;
      if (key < nk) {
        kk = reinterpret_cast<const float4*>(kb + (size_t)key * kvrs)[c];
        vv = reinterpret_cast<const float4*>(vb + (size_t)key * kvrs)[c];
      }
      sk[idx] = kk;
      sv[idx] = vv;
    }
    __syncthreads();
    if (!live) continue;
    const int jn = min(BN, nk - kv0);
    // Each key's K row, then its V row, is read into registers in one batch
    // (a lone wave would otherwise wait out each LDS read in turn).
    for (int j = wv; j < jn; j += NWV) {
      const int key = kv0 + j;
      if (causal && key > pos) break;
      if (W > 0 && key <= pos - W) continue;
      float4 kr[D / 4];
#pragma unroll
      for (int c = 0; c < D / 4; c++) kr[c] = sk[j * (D / 4) + c];
      // four independent partial sums: the dependent FMA chain is D / 4 long
      float d4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < D / 4; c++) {
        d4[0] = fmaf(qr[4 * c], kr[c].x, d4[0]);
        d4[1] = fmaf(qr[4 * c + 1], kr[c].y, d4[1]);
        d4[2] = fmaf(qr[4 * c + 2], kr[c].z, d4[2]);
        d4[3] = fmaf(qr[4 * c + 3], kr[c].w, d4[3]);
      }
      float s = ((d4[0] + d4[1]) + (d4[2] + d4[3])) * scale;
      if (mrow) {
        s += mrow[key];
        if (!(s > -INFINITY)) continue;  // a masked key: no weight (and no -inf - -inf)
      }
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
      for (int c = 0; c < D / 4; c++) kr[c] = sv[j * (D / 4) + c];  // the V row, in K's registers
      const float* vr = reinterpret_cast<const float*>(kr);
#pragma unroll
      for (int d = 0; d < D; d++) acc[d] = fmaf(p, vr[d], acc[d]);
    }
  }
  // Waves 1.. hand their (m, l, acc) to wave 0 through LDS ([wave - 1][D + 2][lane]),
  // which folds them in in wave order.
  __syncthreads();  // every wave is done with the last tile
  float* const ms = reinterpret_cast<float*>(sh);
  if (wv > 0) {
    float* my = ms + (size_t)(wv - 1) * (D + 2) * 64 + lane;
    my[0] = m;
    my[64] = l;
#pragma unroll
    for (int d = 0; d < D; d++) my[(2 + d) * 64] = acc[d];
  }
  __syncthreads();
  if (wv > 0 || !live) return;
  for (int w2 = 1; w2 < NWV; w2++) {
    const float* ot = ms + (size_t)(w2 - 1) * (D + 2) * 64 + lane;
    const float m2 = ot[0], l2 = ot[64], M = fmaxf(m, m2);
    const float a0 = m > -INFINITY ? expf(m - M) : 0.f, a1 = m2 > -INFINITY ? expf(m2 - M) : 0.f;
    l = l * a0 + l2 * a1;
#pragma unroll
    for (int d = 0; d < D; d++) acc[d] = acc[d] * a0 + ot[(2 + d) * 64] * a1;
    m = M;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float* op = out + ((size_t)b * Sq + i) * qrs + (size_t)h * D;
#pragma unroll
  for (int d = 0; d < D; d++) op[d] = acc[d] * inv;
}

hipError_t launch_prefill_f32(const float* q, const float* k, const float* v, float* out, int B, int Sq, int Hq,
                              int Hkv, int D, bool causal, float scale, const KvSpec& kv, const float* q_rope,
                              hipStream_t st) {
  const dim3 grid((unsigned)(B * Hq), (unsigned)((Sq + 63) / 64)), block(64 * kF32Waves);
  if (D == 64)
    hipLaunchKernelGGL(prefill_f32_kernel<64>, grid, block, 0, st, q, k, v, out, Sq, Hq, Hkv, (int)causal, scale, kv,
                       q_rope);
  else
    hipLaunchKernelGGL(prefill_f32_kernel<128>, grid, block, 0, st, q, k, v, out, Sq, Hq, Hkv, (int)causal, scale,
                       kv, q_rope);
  return hipGetLastError();
}

}  // namespace rcgqa
