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
#include <mutex>

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

// Pass 1, bf16 form, on matrix cores.  One workgroup = DW waves handles one
// split of kch keys (2048, or 4096 on large grids) of one (batch, KV head)
// for all G <= 16 query heads of the group, so each K/V row is read from HBM
// once per group.  Each wave streams
// its own 32-key tiles (tiles w, w+DW, ... of the split) through a private LDS
// region, with the next tile prefetched into registers while the current one
// is computed; waves never wait for each other until the final combine.  The
// cache is read with non-temporal loads: it is streamed once per call, so
// keeping it out of L2 / Infinity Cache leaves them to the partial states.
// 8 waves and non-temporal loads were picked by a sweep on the B=64 Hq=64
// Hkv=8 D=128 workload with lengths in [512, 8192]: 512/4/temporal 242 us,
// 1024/8/temporal 235 us, 2048/8/non-temporal 208 us (the split length is
// chosen at launch, see launch_decode_bf16).
//   S^T (32 keys x 16 heads) = K Q^T   v_mfma_f32_16x16x32_bf16, K from LDS
//   O^T (D x 16 heads)      += V^T P^T  same MFMA, V^T via the LDS transpose read
// In both outputs a lane owns one head (lane % 16), so the online-softmax
// rescale is one multiply per accumulator.  The DW waves' states are combined
// in LDS and written as one partial state per (split, head).
namespace {
constexpr int KCH = 2048;  // keys per split, the shorter length (>= KC, so the workspace bound holds)
constexpr int KCH_LONG = 2 * KCH;  // keys per split when the grid stays large (see the launcher)
constexpr long long kDecodeLongSplitGroups = 512;  // two workgroups per CU of the 256
constexpr int TK = 32;     // keys per wave tile
constexpr int DW = 8;      // waves per workgroup
static_assert(KCH >= KC && KCH % TK == 0 && KCH_LONG % TK == 0, "split must be a multiple of the tile and at least KC");
}

template <int D>
__global__ __launch_bounds__(64 * DW) void decode_mfma_kernel(const bf16* __restrict__ q,
                                                             const bf16* __restrict__ kc,
                                                             const bf16* __restrict__ vc,
                                                             const int32_t* __restrict__ kv_lens,
                                                             float* __restrict__ ws, int Hq, int Hkv, int max_kv,
                                                             int nsplit, int kch, float c_log2) {
  constexpr int CH = D / 8;         // 16-byte chunks per row
  constexpr int SW = CH - 1;        // swizzle mask
  constexpr int KSTEP = D / 32;     // k-steps of Q K^T
  constexpr int DBLK = D / 16;      // 16-wide output blocks
  constexpr int LD_PER_LANE = TK * CH / 64;  // 16-byte loads per lane per tile (K or V)
  constexpr int WAVE_LDS = 2 * TK * D;       // bf16 elements per wave (K + V tile)
  __shared__ __attribute__((aligned(16))) bf16 lds[DW * WAVE_LDS];

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int L = min(max(kv_lens[b], 0), max_kv);
  const int k0 = split * kch;
  if (k0 >= L) return;  // uniform: nothing in this split
  const int kend = min(L, k0 + kch);
  const int ntile = (kend - k0 + TK - 1) / TK;
  const int G = Hq / Hkv;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 15, g = lane >> 4;  // head column / lane group of the 16x16 layouts
  bf16* sk = lds + w * WAVE_LDS;
  bf16* sv = sk + TK * D;
  const size_t head_base = ((size_t)b * Hkv + kvh) * (size_t)max_kv * D;
  const bf16* kb = kc + head_base;
  const bf16* vb = vc + head_base;

  // Q^T operand: lane holds q[head n][32 ks + 8 g .. +7]; heads >= G are zero
  bf16x8 qf[KSTEP];
  {
    const bool hv = n < G;
    const bf16x8* src = reinterpret_cast<const bf16x8*>(q + ((size_t)b * Hq + kvh * G + (hv ? n : 0)) * D);
#pragma unroll
    for (int ks = 0; ks < KSTEP; ks++) qf[ks] = hv ? src[4 * ks + g] : bf16x8{};
  }

  f32x4 o[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; i++) o[i] = f32x4{};
  float m_run = -INFINITY, l_run = 0.f;

  // register prefetch of one tile: lane loads chunk (lane % CH) of rows lane / CH + (64 / CH) * p
  bf16x8 pk[LD_PER_LANE], pv[LD_PER_LANE];
  auto load_tile = [&](int t)  __attribute__((always_inline)) {
    const int t0 = k0 + t * TK;
#pragma unroll
    for (int p = 0; p < LD_PER_LANE; p++) {
      const int idx = p * 64 + lane, r = idx / CH, c = idx - r * CH;
      const int key = t0 + r;
      if (key < kend) {
        pk[p] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(kb + (size_t)key * D) + c);
        pv[p] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(vb + (size_t)key * D) + c);
      } else {
        pk[p] = bf16x8{};
        pv[p] = bf16x8{};
      }
    }
  };
  auto store_tile = [&]()  __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < LD_PER_LANE; p++) {
      const int idx = p * 64 + lane, r = idx / CH, c = idx - r * CH;
      const int off = r * D + ((c ^ (row_swizzle(r) & SW)) << 3);
      *reinterpret_cast<bf16x8*>(sk + off) = pk[p];
      *reinterpret_cast<bf16x8*>(sv + off) = pv[p];
    }
  };

  // V transpose-read addressing (fixed per lane): rows 4g + r/4 (+16), cols 16 db + 4 (r % 4)
  const int r16 = lane & 15;
  const int vr1 = 4 * g + (r16 >> 2), vr2 = vr1 + 16;
  const int vcb = 4 * (r16 & 3);

  int t = w;
  if (t < ntile) load_tile(t);
  for (; t < ntile; t += DW) {
    __builtin_amdgcn_wave_barrier();
    store_tile();
    __builtin_amdgcn_wave_barrier();
    if (t + DW < ntile) load_tile(t + DW);
    const int t0 = k0 + t * TK;

    f32x4 s[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; kb2++) {
      s[kb2] = f32x4{};
      const int r = 16 * kb2 + n;
#pragma unroll
      for (int ks = 0; ks < KSTEP; ks++) {
        const int c = 4 * ks + g;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(sk + r * D + ((c ^ (row_swizzle(r) & SW)) << 3));
        s[kb2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[ks], s[kb2], 0, 0, 0);
      }
    }
    // lane holds keys t0 + 16 kb2 + 4 g + j for head n
    float mx = -INFINITY;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; kb2++) {
#pragma unroll
      for (int j = 0; j < 4; j++) {
        float x = s[kb2][j] * c_log2;
        if (t0 + 16 * kb2 + 4 * g + j >= kend) x = -INFINITY;
        s[kb2][j] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = half_swap_max(mx);
    const float m_new = fmaxf(m_run, mx);  // finite: every tile holds a valid key
    const float alpha = fast_exp2(m_run - m_new);
    // weights rounded to bf16 for the P.V product; the row sum adds those
    // same rounded weights, so the normaliser matches what was accumulated
    bf16x8 pf;
    float psum = 0.f;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; kb2++) {
#pragma unroll
      for (int j = 0; j < 4; j++) {
        pf[4 * kb2 + j] = (bf16)fast_exp2(s[kb2][j] - m_new);
        psum += (float)pf[4 * kb2 + j];
      }
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < DBLK; db++) {
      o[db] *= alpha;
      const int cc = 16 * db + vcb;
      const bf16* p1 = sv + vr1 * D + (((cc >> 3) ^ (row_swizzle(vr1) & SW)) << 3) + (cc & 7);
      const bf16* p2 = sv + vr2 * D + (((cc >> 3) ^ (row_swizzle(vr2) & SW)) << 3) + (cc & 7);
      const bf16x8 a = cat8(lds_read_tr16(p1), lds_read_tr16(p2));
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf, o[db], 0, 0, 0);
    }
  }

  // per-wave state of head n: m_run (same in all 4 lane groups), l summed over groups
  l_run += __shfl_xor(l_run, 16);
  l_run = half_swap_sum(l_run);

  // combine the waves in LDS: [w][16 heads][D + 2] fp32 (m, l, acc[D]).  The
  // rows stay 8-byte aligned, so each lane's accumulator run goes out in
  // 8-byte stores (an odd stride, tried to spread the banks, split them into
  // 4-byte stores and measured more LDS instructions and more conflict
  // cycles); the readers take consecutive columns.
  __syncthreads();
  float* st = reinterpret_cast<float*>(lds);
  constexpr int SR = D + 2;
  static_assert(DW * 16 * SR * sizeof(float) <= sizeof(lds), "combine area");
  float* mine = st + (w * 16 + n) * SR;
  if (g == 0) {
    mine[0] = m_run;
    mine[1] = l_run;
  }
#pragma unroll
  for (int db = 0; db < DBLK; db++)
#pragma unroll
    for (int j = 0; j < 4; j++) mine[2 + 16 * db + 4 * g + j] = o[db][j];
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += 64 * DW) {
    const int hh = idx / D, d = idx - hh * D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < DW; ww++) M = fmaxf(M, st[(ww * 16 + hh) * SR]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int ww = 0; ww < DW; ww++) {
      const float* sw = st + (ww * 16 + hh) * SR;
      const float e = sw[1] > 0.f ? fast_exp2(sw[0] - M) : 0.f;
      den = fmaf(e, sw[1], den);
      num = fmaf(e, sw[2 + d], num);
    }
    float* dst = ws + (((size_t)b * Hq + kvh * G + hh) * nsplit + split) * (D + 2);
    dst[2 + d] = num;
    if (d == 0) {
      dst[0] = M;
      dst[1] = den;
    }
  }
}

// Merge of the bf16 pass: the partial maxima are in the log2 domain (scores
// pre-multiplied by scale * log2(e)).  Splits are taken in batches of MB whose
// loads are all issued before the batch is folded in (online, fixed order),
// so the pass is bound by bandwidth rather than by one load latency per split.
template <int D>
__global__ __launch_bounds__(D) void decode_merge2_kernel(const float* __restrict__ ws,
                                                          const int32_t* __restrict__ kv_lens, bf16* __restrict__ out,
                                                          int Hq, int max_kv, int nsplit, int kch) {
  constexpr int MB = 8;
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int L = min(max(kv_lens[b], 0), max_kv);
  const int ns = (L + kch - 1) / kch;
  const float* src = ws + ((size_t)b * Hq + h) * nsplit * (D + 2);
  float M = -INFINITY, den = 0.f, num = 0.f;
  for (int c0 = 0; c0 < ns; c0 += MB) {
    float m[MB], l[MB], a[MB];
#pragma unroll
    for (int i = 0; i < MB; i++) {
      const bool ok = c0 + i < ns;
      const float* p = src + (size_t)(ok ? c0 + i : 0) * (D + 2);
      m[i] = ok ? p[0] : -INFINITY;
      l[i] = ok ? p[1] : 0.f;
      a[i] = ok ? p[2 + d] : 0.f;
    }
    float mb = m[0];
#pragma unroll
    for (int i = 1; i < MB; i++) mb = fmaxf(mb, m[i]);
    const float mn = fmaxf(M, mb);            // finite: split c0 holds a valid key
    const float sc = fast_exp2(M - mn);       // 0 on the first batch
    den *= sc;
    num *= sc;
#pragma unroll
    for (int i = 0; i < MB; i++) {
      const float e = fast_exp2(m[i] - mn);   // 0 for the padding entries
      den = fmaf(e, l[i], den);
      num = fmaf(e, a[i], num);
    }
    M = mn;
  }
  out[((size_t)b * Hq + h) * D + d] = (bf16)(ns > 0 ? num / den : 0.f);
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

template <int D>
static void launch_decode_bf16(const void* q, const void* kc, const void* vc, const int32_t* kv_lens, void* out,
                               int B, int Hq, int Hkv, int max_kv, float scale, void* ws, hipStream_t st) {
  // Longer splits halve the partial states and the workgroups' fixed costs,
  // but each workgroup (one per CU: its LDS takes most of a CU's) then
  // streams twice the keys, so they are taken only while the grid keeps at
  // least two workgroups per CU.  On B=64 Hq=64 Hkv=8 D=128 with lengths in
  // [512, 8192]: 1024 keys 5830 GB/s, 2048 6030, 3072 6020, 4096 6100, 6144 4740.
  const int kch = (long long)B * Hkv * ((max_kv + KCH_LONG - 1) / KCH_LONG) >= kDecodeLongSplitGroups ? KCH_LONG : KCH;
  const int nsplit = (max_kv + kch - 1) / kch;
  const float c_log2 = (float)((double)scale * 1.4426950408889634);
  hipLaunchKernelGGL(decode_mfma_kernel<D>, dim3(nsplit, Hkv, B), dim3(64 * DW), 0, st, (const bf16*)q,
                     (const bf16*)kc, (const bf16*)vc, kv_lens, (float*)ws, Hq, Hkv, max_kv, nsplit, kch, c_log2);
  hipLaunchKernelGGL(decode_merge2_kernel<D>, dim3(Hq, B), dim3(D), 0, st, (const float*)ws, kv_lens, (bf16*)out, Hq,
                     max_kv, nsplit, kch);
}

hipError_t launch_decode(const void* q, const void* kc, const void* vc, const int32_t* kv_lens, void* out, int B,
                         int Hq, int Hkv, int D, int max_kv, float scale, bool bf16_io, void* ws, hipStream_t st) {
  if (bf16_io) {
    if (D == 64) launch_decode_bf16<64>(q, kc, vc, kv_lens, out, B, Hq, Hkv, max_kv, scale, ws, st);
    else launch_decode_bf16<128>(q, kc, vc, kv_lens, out, B, Hq, Hkv, max_kv, scale, ws, st);
  } else {
    if (D == 64) launch_decode_t<float, 64>(q, kc, vc, kv_lens, out, B, Hq, Hkv, max_kv, scale, ws, st);
    else launch_decode_t<float, 128>(q, kc, vc, kv_lens, out, B, Hq, Hkv, max_kv, scale, ws, st);
  }
  return hipGetLastError();
}

// Scratch of the no-allocation decode entry point: the split-K partial states
// live in this fixed array instead of a caller-owned workspace.  Every GPU the
// library runs on holds its own copy for the life of the process.  In host
// code `scratch` names a host-side stand-in, never a device address: the
// device address is looked up once per device and only that pointer is used.
static __device__ __align__(256) float scratch[kDecodeNoAllocBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};
}  // namespace

size_t decode_scratch_bytes(int B, int Hq, int D, int max_kv, bool bf16_io) {
  const size_t per = bf16_io ? KCH : KC;  // keys per partial state in the bf16 / fp32 pass
  const size_t n = ((size_t)max_kv + per - 1) / per;
  return (size_t)B * Hq * n * (size_t)(D + 2) * sizeof(float);
}

hipError_t decode_noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // the current device's copy
    if (e != hipSuccess) return e;
    g_scratch_dev[dev] = p;
  }
  *ptr = g_scratch_dev[dev];
  return hipSuccess;
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
