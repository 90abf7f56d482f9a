// bf16 prefill attention on CDNA4 matrix cores (gfx950).
//
// Method: "【HuggingFace Transformers】LlamaAttention源码解析", section 1.2 steps 2-4
// and section 2 steps 4-5: scores = scale * Q K^T, additive causal mask,
// softmax kept in fp32 (also "Llama2 Transformer架构解析与优化实践" section 3.2),
// weights @ V; query head h reads K/V head h / G (repeat_kv).
//
// Design (one workgroup = NW waves = 32 NW query rows of one (batch, head);
// NW = 8 when the grid is large enough, else 4; grids too small for that run
// one 8-wave workgroup per CU split into two or four key groups, see the
// launcher):
//  * K/V tiles of 64 keys (32 with four key groups) are double-buffered in
//    LDS and filled with direct global->LDS loads (buffer / global load ...
//    lds) one tile ahead of the math, with a row-dependent XOR swizzle of
//    16-byte chunks so all three read patterns below are bank-conflict free.
//    One barrier per tile.
//  * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    K rows are the A operand (read straight from LDS), the wave's 32 query
//    rows are the B operand (held in registers for the whole kernel).  In the
//    output layout every lane then owns ONE query row (lane % 32) and 32 of
//    the tile's 64 keys; the other 32 sit in lane ^ 32, so row max / row sum
//    need one v_permlane32_swap and no LDS.
//  * Online softmax in the exp2 domain with fp32 running max / sum per lane.
//    The query registers carry scale * log2(e) (rounded to bf16), and each
//    tile's Q K^T product starts from the accumulator value -m_ref, the row's
//    reference max, so the weights are a bare exp2 of the product.  The
//    reference only moves when a row's max grows by more than 2^8 (lazy
//    rescale), so the O rescale is skipped on almost every tile.
//  * O^T = V^T P^T, again 32x32x16: P^T comes straight from the score
//    registers (converted to bf16; the MFMA's k index is permuted to match the
//    score layout), V^T is read from the row-major V tile with the gfx950 LDS
//    transpose read (ds_read_b64_tr_b16).  O^T keeps the query row on the lane,
//    so the rescale by exp2(m_old - m_new) is one multiply per accumulator.
//  * Causal: tiles past the block's last row are never loaded; a wave skips
//    the math of tiles past its own last row; only diagonal / tail tiles pay
//    for per-element masking.  Heaviest query tiles are dispatched first.
//  * The same kernel serves chunked / variable-length prefill against a cache
//    (keys through strides, per-sequence key counts, queries aligned to the
//    end of their sequence) and the causal sliding window, whose tiles
//    before the block's first window are never loaded either.
//  * Given a per-token cos/sin table (written by the RoPE kernel while it
//    rotates the keys), each lane rotates its query row in registers before
//    the first tile ("LLaMA2大语言模型架构详解", section "Rotary Position
//    Encoding"), so the queries never make a separate pass through memory.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "grid_model.h"
#include "launch.h"

namespace rcgqa {

namespace {
constexpr float kRescaleLog2 = 8.f;      // lazy rescale threshold (log2 units)
constexpr int PREF = 4;                  // K-operand LDS reads kept ahead of the MFMAs
// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x008, kSchedDsRead = 0x100;
}  // namespace

// Direct global->LDS tile loads, 16 bytes per lane, landing at l + 16 * lane.
//
// They are written as inline asm rather than through the load-to-LDS
// builtins on purpose.  The compiler's wait-count pass cannot tell the LDS
// transpose reads (ds_read_b64_tr_b16, whose builtin carries no alias
// information) apart from the tile being loaded, so with the builtins it puts
// a wait for every load in flight in front of the first transpose read of
// each tile: the P.V operands could then not be read before the next tile's
// loads had landed.  Here completion is waited for explicitly, with a full
// s_waitcnt before the per-tile barrier, and nothing reads a buffer that has
// loads in flight before that barrier.  Each asm sets M0 (the LDS address of
// the wave's 64 x 16 bytes) and leaves the one wait state the hardware needs
// before the load reads it; nothing else in this kernel uses M0.
__device__ __forceinline__ void lds_dma16(const void* g, bf16* l) {
  const uint32_t m = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) void*)l);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m));
}

// The same load through a buffer descriptor: the tile's base lives in scalar
// registers and the per-lane byte offset `voff` is fixed for the whole
// kernel, so issuing a tile takes no vector address arithmetic.  The
// descriptor is raw (unstrided) with the largest range: every offset used is
// inside the tensor by construction.  The last word is the gfx9-family buffer
// format for untyped dword access.
__device__ __forceinline__ void lds_buf16(const void* base, uint32_t voff, bf16* l) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  const uint64_t p = (uint64_t)base;
  const i32x4 rs = {(int)(uint32_t)p, (int)((p >> 32) & 0xffff), (int)0xFFFFFFFF, 0x00020000};
  const uint32_t m = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) void*)l);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rs),
               "s"(m));
}

// Stream-K state of one launch (SPL kernels only; see grid::stream_ranges):
// one counter per query tile at cnt, partial O blocks of BM x D fp16 values
// at o (pairs packed in 32-bit words, in the accumulator layout: [wave]
// [register pair][lane]), the (reference max, row sum, O scale, unused)
// rows [slot][BM][4] at ml; the plan's units per (batch, head); the first
// unit of every query tile of a (batch, head) block in list order
// (tstart[nqt] = per) and of every workgroup (wstart[G] = all units); per
// workgroup the list index of the tile holding its first unit, the
// workgroup holding that tile's first unit and the one holding the last
// unit of the tile its range ends in.  All computed on the host.
constexpr int kStreamMaxTiles = 128;  // query tiles per (batch, head): S up to 32768
constexpr int kStreamMaxGroups = 256;
struct SplitArgs {
  uint32_t* o;
  float* ml;
  int* cnt;
  int per;
  int tstart[kStreamMaxTiles + 1];
  int wstart[kStreamMaxGroups + 1];
  uint16_t wtile[kStreamMaxGroups];
  uint8_t wlo[kStreamMaxGroups], whi[kStreamMaxGroups];
};

// GEN: keys through per-sequence counts (query rows aligned to the end of
// their sequence) and an optional sliding window; without it every sequence
// has Sq keys, queries and keys aligned, and the bounds fold to constants.
// KSPLIT > 1: the NW waves form KSPLIT groups that take the same 32*NW/KSPLIT
// query rows over consecutive parts of the key range, each with its own LDS
// tiles, and merge their softmax states through LDS at the end (more waves in
// flight for grids too small to fill the GPU, with no memory outside the
// workgroup).  BNT keys per K/V tile: 64, or 32 so that four groups' double
// buffers fit in LDS.
// MSK: an additive mask (kv.mask, plain layout) is added to the scores; each
// lane loads its row's values for the next tile while the current one runs.
// SPL: stream-K over workgroups (causal, no cache or mask): workgroup w runs
// a range of units of the causal work (grid::stream_plan), which may cross
// query tiles; a piece of a tile that other workgroups share writes its
// (O, m_ref, l) rows to the split workspace, and the workgroup that completes
// the tile's count merges the pieces in key order and writes the rows (no
// workgroup ever waits for another).
template <int D, int NW, bool GEN, int KSPLIT, int BNT, bool MSK, bool SPL = false>
__global__ __launch_bounds__(64 * NW, 2) void prefill_bf16_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                             const bf16* __restrict__ v, bf16* __restrict__ out,
                                                             int Sq, int Hq, int Hkv, int causal, float c_log2,
                                                             int nqt, int npairs, KvSpec kv,
                                                             const float* __restrict__ q_rope, SplitArgs sp) {
  constexpr int BN = BNT;           // keys per K/V tile
  constexpr int NKB = BN / 32;      // 32-key blocks per tile
  constexpr int NWG = NW / KSPLIT;  // waves per key group
  constexpr int BM = 32 * NWG;      // query rows per workgroup (32 per wave of a group)
  constexpr int KS = D / 16;  // k-steps of the Q K^T contraction
  constexpr int DB = D / 32;  // 32-wide blocks of the output head dim
  constexpr int CH = D / 8;   // 16-byte chunks per row
  constexpr int SW = CH - 1;  // swizzle mask
  static_assert(CH <= 16 && (CH & (CH - 1)) == 0, "D must be 64 or 128");
  constexpr int TILE = BN * D;              // elements of one K (or V) tile
  constexpr int ROWS_PER_LD = 64 / CH;      // rows one wave-wide 16-byte load fills
  constexpr int LD_PER_WAVE = BN / NWG / ROWS_PER_LD;
  static_assert(LD_PER_WAVE >= 1, "tile rows per wave");
  // With a mask on the 8-wave unsplit grid, mask tiles [BM rows][BN keys] are
  // double-buffered in LDS after the K/V buffers.
  constexpr bool MSTAGE = MSK && NW == 8 && KSPLIT == 1;
  constexpr int MTILE = MSTAGE ? 32 * NW * BN : 0;
  __shared__ __attribute__((aligned(16))) bf16 lds[KSPLIT * 2 * 2 * TILE + 2 * MTILE];  // [group][buffer][K | V][BN][D]
  __shared__ int split_last;  // SPL: this workgroup completed its tile's count

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int grp = KSPLIT > 1 ? wu / NWG : 0, wr = KSPLIT > 1 ? wu % NWG : wu;  // key group; rows slot
  bf16* const ldsg = lds + grp * 2 * 2 * TILE;
  const int col = lane & 31, hf = lane >> 5;
  // Work item of this workgroup.  The work list is ordered (batch, query head,
  // query-tile slot), so consecutive items share a head and consecutive heads
  // share a KV head.  The hardware hands consecutive workgroup ids to the 8
  // XCDs in turn; each XCD is given one contiguous eighth of the list, so the
  // query tiles (and GQA heads) that reuse a K/V stream run on one XCD and
  // hit its L2.  A slot is either one query tile or, when there are enough
  // workgroups to fill the GPU (npairs < nqt), the pair (nqt-1-p, p): a
  // heavy and a light causal tile, so every workgroup does the same work.
  // (Stream-K workgroups take contiguous unit ranges per XCD the same way.)
  const int total = (int)gridDim.x;
  const int wid = (int)blockIdx.x;
  const int item = (total & 7) == 0 ? (wid & 7) * (total >> 3) + (wid >> 3) : wid;
  const size_t qrs = (size_t)Hq * D, kvrs = (size_t)kv.sr;
  // One query tile of (batch, head) bh at rows [q0, q0 + BM).  SPL: key tiles
  // [seg_lo, seg_hi) of the tile, which the plan gives seg_n key tiles (a
  // sequence shorter than the plan assumes has fewer visible ones; the rest
  // are skipped) and which starts at unit seg_t0, has counter seg_tile and
  // one piece in each of workgroups seg_w0..seg_w1; this workgroup's range
  // starts at unit seg_a.
  auto run_qtile = [&](const int q0, const int bh, const int seg_lo, const int seg_hi, const int seg_n, const int seg_t0,
                       const int seg_tile, const int seg_w0, const int seg_w1,
                       const int seg_a) __attribute__((always_inline)) {
  const int b = bh / Hq, h = bh - b * Hq;
  const int kvh = h / (Hq / Hkv);
  const bf16* kb = k + (size_t)b * kv.sb + (size_t)kvh * kv.sh;
  const bf16* vb = v + (size_t)b * kv.sb + (size_t)kvh * kv.sh;
  // this sequence's keys; query i sits at absolute position i + off
  const int nkeys = GEN ? min(max(kv.lens[b], 0), kv.max_kv) : Sq;
  const int off = GEN ? nkeys - Sq : 0, W = GEN ? kv.window : 0;

  const int qrow = q0 + wr * 32 + col;  // this lane's query row
  bf16x8 qf[KS];
  if (qrow < Sq) {
    const bf16x8* src = reinterpret_cast<const bf16x8*>(q + ((size_t)b * Sq + qrow) * qrs + (size_t)h * D);
#pragma unroll
    for (int ks = 0; ks < KS; ks++) qf[ks] = src[2 * ks + hf];
  } else {
#pragma unroll
    for (int ks = 0; ks < KS; ks++) qf[ks] = bf16x8{};
  }
  // Cos/sin of the row's token when the queries still need their rotation
  // (applied after the first tile's barrier, so these loads, the query loads
  // and the first tile's direct loads are all in flight together).
  f32x4 rc[KS / 2][2], rs[KS / 2][2];
  const bool rot = q_rope && qrow < Sq;
  if (rot) {
    const float* cs = q_rope + ((size_t)b * Sq + qrow) * D;
#pragma unroll
    for (int ks = 0; ks < KS / 2; ks++) {
      const int i0 = 16 * ks + 8 * hf;
      rc[ks][0] = *reinterpret_cast<const f32x4*>(cs + i0);
      rc[ks][1] = *reinterpret_cast<const f32x4*>(cs + i0 + 4);
      rs[ks][0] = *reinterpret_cast<const f32x4*>(cs + D / 2 + i0);
      rs[ks][1] = *reinterpret_cast<const f32x4*>(cs + D / 2 + i0 + 4);
    }
  }

  // Additive mask: this lane's 2 NKB runs of 4 consecutive keys per tile (the
  // score layout).  On the 8-wave unsplit grid (which the launcher uses for
  // masks only when their rows hold a multiple of 8 entries) each tile's
  // [BM][BN] block comes into LDS with the K/V tiles by direct loads (16-byte
  // chunks; chunk c of block row r sits at chunk c ^ ((r >> 1) & 7), which
  // spreads a wave's per-row reads over the banks).  The other grids read
  // each lane's row from memory one tile ahead, into one register set per
  // tile buffer; rows past Sq read nothing and keys past the sequence read
  // zeros (they are masked anyway).
  constexpr bool mstage = MSTAGE;
  bf16* const mlds = lds + KSPLIT * 2 * 2 * TILE;
  auto issue_mask = [&](int t, int buf) __attribute__((always_inline)) {
    if constexpr (MSTAGE) {
      constexpr int LDM = BM * BN * (int)sizeof(bf16) / 1024 / NW;  // 1 KB direct loads per wave
      const bf16* mb = reinterpret_cast<const bf16*>(kv.mask) + (size_t)b * kv.msb + (size_t)h * kv.msh;
#pragma unroll
      for (int i = 0; i < LDM; i++) {
        const int r0 = (wr * LDM + i) * 8;  // 8 block rows of BN keys per load
        const int r = r0 + lane / 8, c = (lane % 8) ^ ((r >> 1) & 7);
        const int row = min(q0 + r, Sq - 1);
        const int key = min(t * BN + c * 8, (int)kv.msr - 8);  // inside the row; keys past Sq are masked
        lds_dma16(mb + (size_t)row * kv.msr + key, mlds + buf * MTILE + r0 * BN);
      }
    }
  };
  bf16x4 mk[MSK ? 2 : 1][NKB][4];
  const bf16* mrow = nullptr;
  if constexpr (MSK) {
    if (qrow < Sq)
      mrow = reinterpret_cast<const bf16*>(kv.mask) + (size_t)b * kv.msb + (size_t)h * kv.msh + (size_t)qrow * kv.msr;
  }
  const bool mvec = (kv.msr & 3) == 0;  // 8-byte aligned runs (the base is 16-byte aligned)
  auto load_mask = [&](int t, int set) __attribute__((always_inline)) {
    if constexpr (mstage) return;
#pragma unroll
    for (int kb2 = 0; kb2 < NKB; kb2++)
#pragma unroll
      for (int g4 = 0; g4 < 4; g4++) {
        const int key = t * BN + kb2 * 32 + 8 * g4 + 4 * hf;
        bf16x4 m4 = {};
        if (mrow) {
          if (mvec && key + 4 <= nkeys) {
            m4 = *reinterpret_cast<const bf16x4*>(mrow + key);
          } else {
#pragma unroll
            for (int c = 0; c < 4; c++)
              if (key + c < nkeys) m4[c] = mrow[key + c];
          }
        }
        mk[set][kb2][g4] = m4;
      }
  };
  constexpr float kLog2e = 1.4426950408889634f;  // the mask enters the log2-unit scores as mask * log2(e)

  // Tile loader: wave wr of a group fills tile rows [wr BN/NWG, (wr+1) BN/NWG) of K and V with
  // direct global->LDS loads.  Lane p of a load lands at physical chunk
  // p % CH of row p / CH, so it fetches the logical chunk that the swizzle
  // puts there.  Keys past Sk are clamped to Sk-1 (finite data; masked later).
  const int lrow = lane / CH, lpc = lane % CH;
  // Byte offsets of this lane's loads inside a tile do not depend on the tile:
  // computed once (32-bit), so a full tile costs one scalar base update and no
  // per-lane address arithmetic.  Only a tile crossing Sk clamps per lane.
  uint32_t loff[LD_PER_WAVE];
#pragma unroll
  for (int i = 0; i < LD_PER_WAVE; i++) {
    const int r = wr * (BN / NWG) + i * ROWS_PER_LD + lrow;
    loff[i] = (uint32_t)(r * (int)kvrs + ((lpc ^ (row_swizzle(r) & SW)) << 3)) * (uint32_t)sizeof(bf16);
  }
  auto issue = [&](int t, int buf)  __attribute__((always_inline)) {
    bf16* kd = ldsg + buf * 2 * TILE;
    bf16* vd = kd + TILE;
    if (t * BN + BN <= nkeys) {
      const bf16* kt = kb + (size_t)t * BN * kvrs;
      const bf16* vt = vb + (size_t)t * BN * kvrs;
#pragma unroll
      for (int i = 0; i < LD_PER_WAVE; i++) {
        const int r0 = wr * (BN / NWG) + i * ROWS_PER_LD;  // wave-uniform
        lds_buf16(kt, loff[i], kd + r0 * D);
        lds_buf16(vt, loff[i], vd + r0 * D);
      }
    } else {
#pragma unroll
      for (int i = 0; i < LD_PER_WAVE; i++) {
        const int r0 = wr * (BN / NWG) + i * ROWS_PER_LD;
        const int r = r0 + lrow;
        const int key = min(t * BN + r, nkeys - 1);
        const size_t goff = (size_t)key * kvrs + (size_t)((lpc ^ (row_swizzle(r) & SW)) << 3);
        lds_dma16(kb + goff, kd + r0 * D);
        lds_dma16(vb + goff, vd + r0 * D);
      }
    }
  };

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; db++) o[db] = f32x16{};
  // Scores are formed in log2 units (the query registers carry scale * log2(e))
  // and relative to the row's reference max m_ref: every tile's Q K^T product
  // starts from the accumulator value -m_ref (negm), so the weights are plain
  // exp2 of the scores.  `lim` is the lazy-rescale threshold on those relative
  // scores; -1e30 marks a row that has not seen a visible key yet (m_ref = 0
  // meanwhile), so a row whose first tiles are fully masked keeps zero weights.
  // (The masked two-group kernel, whose per-lane mask registers leave no room
  // for the 16 offset registers, subtracts m_ref after the product instead.)
  constexpr bool NEGM = !(MSK && KSPLIT == 2);
  float m_ref = 0.f, l_run = 0.f, lim = -1e30f;
  f32x16 negm = {};

  // keys any row of this query tile can see: tiles [t_lo, t_hi)
  const int key_hi = causal ? min(nkeys, q0 + BM + off) : nkeys;
  const int key_lo = (causal && W > 0) ? max(0, q0 + off - W + 1) : 0;
  const int t_lo = key_lo / BN, t_hi = key_hi > 0 ? (key_hi + BN - 1) / BN : 0;
  // this group's tiles [tg_lo, tg_hi) (possibly empty); all groups run `steps` barrier steps.
  // A stream-K piece takes the tiles [seg_lo, seg_hi) of its range (t_lo = 0
  // there), cut at t_hi: against a cache, a sequence shorter than the plan
  // assumes has fewer key tiles, and none past them is ever loaded.
  const int ntl = max(t_hi - t_lo, 0);
  const int tg_lo = SPL ? min(seg_lo, t_hi) : t_lo + grp * ((ntl + KSPLIT - 1) / KSPLIT);
  const int tg_hi = SPL ? min(seg_hi, t_hi) : min(tg_lo + (ntl + KSPLIT - 1) / KSPLIT, t_lo + ntl);
  const int steps = SPL ? tg_hi - tg_lo : (ntl + KSPLIT - 1) / KSPLIT;
  const int wrow_lo = q0 + wr * 32, wrow_hi = wrow_lo + 31;

  // transpose-read addressing of V (fixed per lane)
  const int r16 = lane & 15, g = lane >> 4;
  const int vrow_base = 4 * hf + (r16 >> 2);
  const int vcol_base = 16 * (g & 1) + 4 * (r16 & 3);
  // Per-lane byte offsets of the operand reads inside a tile.  The row block
  // (kb2, kc) and the buffer only add immediates: the swizzle depends on
  // row % 16, which those blocks do not change.
  int koff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ks++)
    koff[ks] = (col * D + (((2 * ks + hf) ^ (row_swizzle(col) & SW)) << 3)) * (int)sizeof(bf16);
  int voff[DB][2];
#pragma unroll
  for (int db = 0; db < DB; db++)
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const int row = vrow_base + 8 * j, cc = 32 * db + vcol_base;
      voff[db][j] = (row * D + (((cc >> 3) ^ (row_swizzle(row) & SW)) << 3) + (cc & 7)) * (int)sizeof(bf16);
    }

  // One tile; `bufc` carries the buffer parity at compile time so every LDS
  // address below is a per-lane constant plus an immediate offset.
  auto tile_step = [&](int t, auto bufc)  __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    const int kv0 = t * BN;
    if (t + 1 < tg_hi) issue(t + 1, buf ^ 1);
    if constexpr (MSK) {
      if (t + 1 < tg_hi) {
        if (mstage) issue_mask(t + 1, buf ^ 1);
        load_mask(t + 1, buf ^ 1);
      }
    }
    // else the whole tile is masked for this wave (past its last row, or before its window),
    // or (second key group, odd tile count) past the group's range
    if (t < tg_hi && !(causal && kv0 > wrow_hi + off) && !(W > 0 && kv0 + BN - 1 <= wrow_lo + off - W)) {
      const bf16* sk = ldsg + buf * 2 * TILE;
      const bf16* sv = sk + TILE;

      // S^T = K Q^T - m_ref: NKB 32-key blocks, chains interleaved, the K
      // operand reads kept PREF products ahead of the MFMAs.
      f32x16 s[NKB];
      constexpr int NP = NKB * KS;  // products of the step, kb2 fastest
      auto kread = [&](int i) __attribute__((always_inline)) {
        return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(sk) + koff[i / NKB] +
                                                (i % NKB) * 32 * D * (int)sizeof(bf16));
      };
      if constexpr (SPL) {
        // Through an explicit ring of PREF registers with a scheduling barrier
        // after each product: in this instantiation the scheduler otherwise
        // moves every read down to its product and waits for each one.
        bf16x8 kring[PREF];
#pragma unroll
        for (int i = 0; i < PREF; i++) kring[i] = kread(i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NP; i++) {
          const int ks = i / NKB, kb2 = i % NKB;
          s[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kring[i % PREF], qf[ks],
                                                           ks > 0 ? s[kb2] : NEGM ? negm : f32x16{}, 0, 0, 0);
          if (i + PREF < NP) kring[i % PREF] = kread(i + PREF);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int i = 0; i < NP; i++) {
          const int ks = i / NKB, kb2 = i % NKB;
          s[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kread(i), qf[ks], ks > 0 ? s[kb2] : NEGM ? negm : f32x16{},
                                                           0, 0, 0);
        }
        if (PREF > 0) {
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, PREF, 0);
#pragma unroll
          for (int i = 0; i < NP - PREF; i++) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, PREF, 0);
        }
      }

      // the first 16-key chunk of P.V operands is read now, so its latency
      // hides under the softmax (the first P.V products then start as soon
      // as the first eight weights exist)
      bf16x8 vpre[DB];
#pragma unroll
      for (int db = 0; db < DB; db++)
        vpre[db] = cat8(lds_read_tr16(reinterpret_cast<const bf16*>(reinterpret_cast<const char*>(sv) + voff[db][0])),
                        lds_read_tr16(reinterpret_cast<const bf16*>(reinterpret_cast<const char*>(sv) + voff[db][1])));
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (!NEGM) {
#pragma unroll
        for (int kb2 = 0; kb2 < NKB; kb2++) s[kb2] -= m_ref;
      }
      if constexpr (MSK) {
        if (mstage) {
          const int rr = wr * 32 + col;  // this lane's row of the block
          const bf16* mt = mlds + buf * MTILE + rr * BN + 4 * hf;
#pragma unroll
          for (int kb2 = 0; kb2 < NKB; kb2++)
#pragma unroll
            for (int g4 = 0; g4 < 4; g4++)
              mk[buf][kb2][g4] = *reinterpret_cast<const bf16x4*>(mt + (((kb2 * 4 + g4) ^ ((rr >> 1) & 7)) * 8));
        }
#pragma unroll
        for (int kb2 = 0; kb2 < NKB; kb2++)
#pragma unroll
          for (int i = 0; i < 16; i++) s[kb2][i] = fmaf((float)mk[buf][kb2][i >> 2][i & 3], kLog2e, s[kb2][i]);
      }
      // mask (diagonal / tail tiles only) and row max
      if ((causal && kv0 + BN - 1 > wrow_lo + off) || kv0 + BN > nkeys || (W > 0 && kv0 <= wrow_hi + off - W)) {
        if constexpr (MSK && !MSTAGE) {
          // (the kernels that keep mask registers per lane: no room for the row bounds)
#pragma unroll
          for (int kb2 = 0; kb2 < NKB; kb2++)
#pragma unroll
            for (int i = 0; i < 16; i++) {
              const int key = kv0 + kb2 * 32 + 8 * (i >> 2) + 4 * hf + (i & 3);
              if (key >= nkeys || (causal && key > qrow + off) || (W > 0 && key <= qrow + off - W))
                s[kb2][i] = -INFINITY;
            }
        } else {
          // this row sees keys base + c for lo <= c <= hi (c: the element's offset in the lane's runs)
          const int base = kv0 + 4 * hf;
          const int hi = (causal ? min(nkeys - 1, qrow + off) : nkeys - 1) - base;
          const int lo = qrow + off - W + 1 - base;
#pragma unroll
          for (int kb2 = 0; kb2 < NKB; kb2++)
#pragma unroll
            for (int i = 0; i < 16; i++) {
              const int c = kb2 * 32 + 8 * (i >> 2) + (i & 3);
              if (c > hi || (W > 0 && c < lo)) s[kb2][i] = -INFINITY;
            }
        }
      }
      float mx = s[0][0];
#pragma unroll
      for (int i = 1; i < 16; i++) mx = fmaxf(mx, s[0][i]);
#pragma unroll
      for (int kb2 = 1; kb2 < NKB; kb2++)
#pragma unroll
        for (int i = 0; i < 16; i++) mx = fmaxf(mx, s[kb2][i]);
      mx = half_swap_max(mx);

      // lazy rescale: move the reference only in rows whose max grew by more
      // than 2^kRescaleLog2 (exact either way: O and l share the reference),
      // or that see their first visible key
      if (__any(mx > lim)) {
        const bool up = mx > lim;
        const float d = up ? mx : 0.f;
        const float alpha = up && lim > -1e29f ? fast_exp2(-mx) : 1.f;  // O = l = 0 before the first key
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; db++) o[db] *= alpha;
        m_ref += d;
        lim = up ? kRescaleLog2 : lim;
        if constexpr (NEGM) {
#pragma unroll
          for (int i = 0; i < 16; i++) negm[i] = -m_ref;
        }
#pragma unroll
        for (int kb2 = 0; kb2 < NKB; kb2++)
#pragma unroll
          for (int i = 0; i < 16; i++) s[kb2][i] -= d;
      }
      bf16x8 pf[2 * NKB];
#pragma unroll
      for (int kb2 = 0; kb2 < NKB; kb2++) {
#pragma unroll
        for (int i = 0; i < 16; i++) pf[kb2 * 2 + (i >> 3)][i & 7] = (bf16)fast_exp2(s[kb2][i]);
      }
      // row sum of the bf16 weights actually fed to the MFMA (two per dot2,
      // two chains, one of them continuing the running sum)
      float sa = l_run, sb = 0.f;
#pragma unroll
      for (int j = 0; j < 2 * NKB; j++)
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
          sa = bf16_pair_sum(pf[j][2 * e], pf[j][2 * e + 1], sa);
          sb = bf16_pair_sum(pf[j][2 * e + 2], pf[j][2 * e + 3], sb);
        }
      l_run = sa + sb;

      // O^T += V^T P^T over the tile's 16-key chunks
#pragma unroll
      for (int kc = 0; kc < 2 * NKB; kc++) {
#pragma unroll
        for (int db = 0; db < DB; db++) {
          const char* vbase = reinterpret_cast<const char*>(sv) + kc * 16 * D * (int)sizeof(bf16);
          const bf16x8 a = kc == 0 ? vpre[db]
                                   : cat8(lds_read_tr16(reinterpret_cast<const bf16*>(vbase + voff[db][0])),
                                          lds_read_tr16(reinterpret_cast<const bf16*>(vbase + voff[db][1])));
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kc], o[db], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of tile t+1 have landed
    __syncthreads();                // ... and everyone's; tile t fully consumed
  };
  if (tg_lo < tg_hi) issue(tg_lo, 0);
  if constexpr (MSK) {
    if (tg_lo < tg_hi) {
      if (mstage) issue_mask(tg_lo, 0);
      load_mask(tg_lo, 0);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (rot) {
    // Rotate the row by its token's cos/sin, with rope_apply's arithmetic.
    // This lane holds elements 16 ks + 8 hf + e; the partner of pair i is
    // i + D/2, i.e. the same e of k-step ks + KS/2 in the same lane.
#pragma unroll
    for (int ks = 0; ks < KS / 2; ks++)
#pragma unroll
      for (int e = 0; e < 8; e++) {
        const float co = rc[ks][e >> 2][e & 3], si = rs[ks][e >> 2][e & 3];
        const float a = (float)qf[ks][e], bb = (float)qf[ks + KS / 2][e];
        qf[ks][e] = (bf16)fmaf(a, co, -(bb * si));
        qf[ks + KS / 2][e] = (bf16)fmaf(bb, co, a * si);
      }
  }
  // The queries carry scale * log2(e), rounded once more to bf16 (after any
  // rotation, so the fused path still equals rotation followed by attention).
#pragma unroll
  for (int ks = 0; ks < KS; ks++)
#pragma unroll
    for (int e = 0; e < 8; e++) qf[ks][e] = (bf16)((float)qf[ks][e] * c_log2);
  for (int i = 0; i < steps; i += 2) {
    tile_step(tg_lo + i, std::integral_constant<int, 0>{});
    if (i + 1 < steps) tile_step(tg_lo + i + 1, std::integral_constant<int, 1>{});
  }
  if constexpr (KSPLIT > 1) {
    static_assert((KSPLIT - 1) * NWG * (DB * 16 + 2) * 64 * sizeof(float) <= sizeof(lds), "hand-over area");
    // Key groups 1.. hand their states to their partner waves of group 0
    // (same rows, same lane layout) through LDS, merged in group order; every
    // tile is consumed and no load is in flight since the last step's barrier.
    constexpr int NV = DB * 16 + 2;
    auto xslot = [&](int g) __attribute__((always_inline)) {
      return reinterpret_cast<float*>(lds) + ((size_t)(g - 1) * NWG + wr) * NV * 64 + lane;
    };
    if (grp > 0) {
      float* xfer = xslot(grp);
#pragma unroll
      for (int db = 0; db < DB; db++)
#pragma unroll
        for (int i = 0; i < 16; i++) xfer[(db * 16 + i) * 64] = o[db][i];
      xfer[(DB * 16) * 64] = lim > -1e29f ? m_ref : -1e30f;  // no visible key: weight 0 in the merge
      xfer[(DB * 16 + 1) * 64] = l_run;
    }
    __syncthreads();
    if (grp == 0) {
      float m0 = lim > -1e29f ? m_ref : -1e30f;
#pragma unroll
      for (int g = 1; g < KSPLIT; g++) {
        const float* xfer = xslot(g);
        const float m1 = xfer[(DB * 16) * 64], l1 = xfer[(DB * 16 + 1) * 64];
        const float m = fmaxf(m0, m1);
        const float a0 = fast_exp2(m0 - m), a1 = fast_exp2(m1 - m);
        l_run = l_run * a0 + l1 * a1;
#pragma unroll
        for (int db = 0; db < DB; db++)
#pragma unroll
          for (int i = 0; i < 16; i++) o[db][i] = o[db][i] * a0 + xfer[(db * 16 + i) * 64] * a1;
        m0 = m;
      }
    }
    __syncthreads();  // the hand-over area is free again before any later tile load
  }

  float l_tot = half_swap_sum(l_run);
  if constexpr (SPL) {
    // workgroups [w0, w1] share this tile; a piece of a shared tile hands its
    // state over (this workgroup's logical index is `item`, its first unit seg_a)
    const int w0 = seg_w0, w1 = seg_w1;
    if (w1 > w0) {
      // The pieces run on any XCD, and each XCD has its own L2, so the
      // hand-over goes through memory without whole-cache maintenance (an L2
      // write-back and invalidate per workgroup measured 4x slower): the
      // state is stored with system-scope stores (written through the L2),
      // this wave waits until they are acknowledged, and only then does the
      // workgroup count itself in with a system-scope atomic.  The workgroup
      // that brings the count to the number of pieces reads the others'
      // states with system-scope loads (served from memory, not from a stale
      // L2 line) issued after it has seen the count, so it sees every store.
      // A row's O goes as fp16 values scaled by the row's largest |O| (so in
      // [-1, 1]; the scale travels in fp32 with m and l), in the accumulators'
      // own layout, register-pair-major ([wave][register pair][lane]), so each
      // store writes 256 contiguous bytes and the merge reads it back into
      // the same waves and lanes.  The merge takes every piece, its own
      // included, in this rounded form and in key order, so the result does
      // not depend on which workgroup merges.
      const int r = wr * 32 + col;
      // slot 2 w for a workgroup's first piece, 2 w + 1 for its last
      const long long me = 2LL * item + (seg_t0 > seg_a ? 1 : 0);
      const float m_me = lim > -1e29f ? m_ref : -1e30f;  // -1e30: no key seen, weight 0 in the merge
      float amax = 0.f;
#pragma unroll
      for (int db = 0; db < DB; db++)
#pragma unroll
        for (int i = 0; i < 16; i++) amax = fmaxf(amax, fabsf(o[db][i]));
      amax = half_swap_max(amax);
      const float sinv = amax > 0.f ? 1.f / amax : 0.f;
      typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));
      uint32_t yw[DB * 8];
#pragma unroll
      for (int db = 0; db < DB; db++)
#pragma unroll
        for (int i = 0; i < 16; i += 2)
          yw[db * 8 + i / 2] =
              __builtin_bit_cast(uint32_t, h16x2{(_Float16)(o[db][i] * sinv), (_Float16)(o[db][i + 1] * sinv)});
      const size_t wl = (size_t)wr * (DB * 8) * 64 + lane;
      uint32_t* po = sp.o + (size_t)me * (BM * D / 2) + wl;
#pragma unroll
      for (int j = 0; j < DB * 8; j++)
        __hip_atomic_store(po + j * 64, yw[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      if (hf == 0) {
        float* pm = sp.ml + ((size_t)me * BM + r) * 4;
        __hip_atomic_store(pm, m_me, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        __hip_atomic_store(pm + 1, l_tot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        __hip_atomic_store(pm + 2, amax, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0) (expcnt, lgkmcnt not waited on): stores acknowledged
      __syncthreads();
      int* const cnt = sp.cnt + seg_tile;
      if (tid == 0)
        split_last = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) == (int)(w1 - w0);
      __syncthreads();
      if (!split_last) return;
      auto ldf = [](const float* p) __attribute__((always_inline)) {
        return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      };
      auto ldw = [](const uint32_t* p) __attribute__((always_inline)) {
        return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      };
      // the tile starts inside workgroup w0's range (its last piece) or at its
      // first unit; for every later workgroup it is the first piece
      const long long s0 = 2LL * w0 + (seg_t0 > sp.wstart[w0] ? 1 : 0);
      auto slot_of = [&](int ww) __attribute__((always_inline)) { return ww == w0 ? s0 : 2LL * ww; };
      float M = -1e30f;
      for (int ww = w0; ww <= w1; ww++) {
        const long long sl = slot_of(ww);
        M = fmaxf(M, sl == me ? m_me : ldf(sp.ml + ((size_t)sl * BM + r) * 4));
      }
      // one piece's (m, l, scale, O words): this workgroup's from registers,
      // the others' from memory; the next piece is fetched while the current
      // one is added in
      uint32_t xw[DB * 8];
      float mc, lc, sc;
      auto fetch = [&](int ww, uint32_t* w, float& m, float& l, float& sca) __attribute__((always_inline)) {
        const long long sl = slot_of(ww);
        if (sl == me) {
          m = m_me;
          l = l_tot;
          sca = amax;
#pragma unroll
          for (int j = 0; j < DB * 8; j++) w[j] = yw[j];
        } else {
          const float* pm = sp.ml + ((size_t)sl * BM + r) * 4;
          m = ldf(pm);
          l = ldf(pm + 1);
          sca = ldf(pm + 2);
          const uint32_t* pc = sp.o + (size_t)sl * (BM * D / 2) + wl;
#pragma unroll
          for (int j = 0; j < DB * 8; j++) w[j] = ldw(pc + j * 64);
        }
      };
      fetch(w0, xw, mc, lc, sc);
      f32x16 acc[DB];
#pragma unroll
      for (int db = 0; db < DB; db++) acc[db] = f32x16{};
      float den = 0.f;
      for (int ww = w0; ww <= w1; ww++) {
        uint32_t nw[DB * 8];
        float mn = 0.f, ln = 0.f, sn = 0.f;
        if (ww < w1) fetch(ww + 1, nw, mn, ln, sn);
        const float e = mc > -1e29f ? fast_exp2(mc - M) : 0.f;
        den = fmaf(e, lc, den);
        const float es = e * sc;
#pragma unroll
        for (int db = 0; db < DB; db++)
#pragma unroll
          for (int i = 0; i < 16; i += 2) {
            const h16x2 y = __builtin_bit_cast(h16x2, xw[db * 8 + i / 2]);
            acc[db][i] = fmaf(es, (float)y[0], acc[db][i]);
            acc[db][i + 1] = fmaf(es, (float)y[1], acc[db][i + 1]);
          }
        mc = mn;
        lc = ln;
        sc = sn;
#pragma unroll
        for (int j = 0; j < DB * 8; j++) xw[j] = nw[j];
      }
#pragma unroll
      for (int db = 0; db < DB; db++) o[db] = acc[db];
      l_tot = den;
      if (tid == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);  // zero for the next call
    }
  }
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (grp == 0 && qrow < Sq) {
    bf16* dst = out + ((size_t)b * Sq + qrow) * qrs + (size_t)h * D;
#pragma unroll
    for (int db = 0; db < DB; db++) {
#pragma unroll
      for (int a = 0; a < 4; a++) {
        const int d = 32 * db + 8 * a + 4 * hf;
        bf16x4 y;
#pragma unroll
        for (int c = 0; c < 4; c++) y[c] = (bf16)(o[db][4 * a + c] * inv);
        *reinterpret_cast<bf16x4*>(dst + d) = y;
      }
    }
  }
  };  // run_qtile
  if constexpr (SPL) {
    // this workgroup's units, piece by piece
    const int u_a = sp.wstart[item], u_end = sp.wstart[item + 1];
    // tiles in list order from the one holding the range's first unit; the
    // first can be shared with earlier workgroups, the last with later ones
    int ti = sp.wtile[item];
    for (int u = u_a; u < u_end; ti++) {
      const int b_ = ti / nqt, j = ti - b_ * nqt;
      const int qt = grid::stream_pair_qt(j, nqt);
      const int t0 = b_ * sp.per + sp.tstart[j], n = sp.tstart[j + 1] - sp.tstart[j], k0 = u - t0;
      const int k_hi = min(n, k0 + (u_end - u));
      const int w0 = t0 < u_a ? (int)sp.wlo[item] : item, w1 = t0 + n > u_end ? (int)sp.whi[item] : item;
      run_qtile(qt * BM, b_, k0, k_hi, n, t0, b_ * nqt + qt, w0, w1, u_a);
      u += k_hi - k0;
    }
  } else {
    const int bh = item / npairs, slot = item - bh * npairs;
    // heavy (late) causal query tiles first: with more workgroups than fit at
    // once, the light ones then fill in behind them
    const int qt_first = (npairs < nqt || causal) ? nqt - 1 - slot : slot;
    run_qtile(qt_first * BM, bh, 0, 0, 0, 0, 0, 0, 0, 0);
    if (npairs < nqt && slot != nqt - 1 - slot) run_qtile(slot * BM, bh, 0, 0, 0, 0, 0, 0, 0, 0);
  }
}

template <int NW, bool GEN, int KSPLIT, int BNT>
static void launch_nw(const void* q, const void* k, const void* v, void* out, int B, int Sq, int Hq, int Hkv,
                      int D, bool causal, float c_log2, int npairs, const KvSpec& kv, const float* q_rope,
                      hipStream_t st) {
  constexpr int BM = 32 * NW / KSPLIT;
  const int nqt = (Sq + BM - 1) / BM;
  const dim3 grid((unsigned)((long long)B * Hq * npairs)), block(64 * NW);
  // masks come with the plain layout only, so GEN kernels have no masked form
  const bool msk = !GEN && kv.mask;
#define RCGQA_PREFILL_LAUNCH(DD, M)                                                                               \
  hipLaunchKernelGGL((prefill_bf16_kernel<DD, NW, GEN, KSPLIT, BNT, M>), grid, block, 0, st, (const bf16*)q,    \
                     (const bf16*)k, (const bf16*)v, (bf16*)out, Sq, Hq, Hkv, (int)causal, c_log2, nqt, npairs, kv, \
                     q_rope, SplitArgs{})
  if (D == 64) {
    if (msk) RCGQA_PREFILL_LAUNCH(64, !GEN);
    else RCGQA_PREFILL_LAUNCH(64, false);
  } else {
    if (msk) RCGQA_PREFILL_LAUNCH(128, !GEN);
    else RCGQA_PREFILL_LAUNCH(128, false);
  }
#undef RCGQA_PREFILL_LAUNCH
}

template <int NW, int KSPLIT, int BNT = 64>
static void launch_nw(const void* q, const void* k, const void* v, void* out, int B, int Sq, int Hq, int Hkv,
                      int D, bool causal, float c_log2, int npairs, const KvSpec& kv, const float* q_rope,
                      hipStream_t st) {
  if (kv.lens || kv.window > 0)
    launch_nw<NW, true, KSPLIT, BNT>(q, k, v, out, B, Sq, Hq, Hkv, D, causal, c_log2, npairs, kv, q_rope, st);
  else
    launch_nw<NW, false, KSPLIT, BNT>(q, k, v, out, B, Sq, Hq, Hkv, D, causal, c_log2, npairs, kv, q_rope, st);
}

namespace {
// The split workspace starts with a fixed block of per-tile counters, so that
// calls of any shape find theirs at the same place (zeroed by the last call);
// the partial states follow it, two slots per workgroup.
constexpr int kSplitCounters = 1024;
constexpr size_t kSplitCounterBytes = kSplitCounters * sizeof(int);
constexpr int kStreamBM = 256;     // 8-wave workgroups, one per CU
constexpr int kStreamMinUnits = 4;  // units per workgroup at least
constexpr int kStreamPieceCost = 2;  // cost of a piece, in units (its prologue)
constexpr int kStreamMergeCost = 3;  // cost of merging a shared tile's pieces, in units
// Whether the launcher pairs heavy and light causal tiles (the 8-wave grid, or
// the 4-wave grid when it has 512 pairs): those grids are as fast as stream-K.
bool paired_grid(long long bh, int Sq) {
  const int nqt8 = (Sq + 255) / 256, nqt4 = (Sq + 127) / 128;
  return (nqt8 > 1 && bh * ((nqt8 + 1) / 2) >= 512) || (nqt4 > 1 && bh * ((nqt4 + 1) / 2) >= 512);
}
// Stream-K is used for causal prefills without a window or mask (plain, or
// against a cache of max_kv >= Sq rows, see below) that the launcher would
// run on an unpaired grid, with at least kStreamMinShare units per workgroup (below
// that the fixed cost of a piece outweighs the balance: 8 heads of 2100 or
// 3000 tokens ran slower than the key-group grids, 8 heads of 4096 and more
// faster).  Against a cache the plan assumes every sequence holds max_kv
// rows (query row i at key position max_kv - Sq + i): shorter sequences
// stay correct and only leave part of their pieces idle.
constexpr int kStreamMinShare = 16;
int stream_off(int Sq, const KvSpec& kv) { return kv.lens ? kv.max_kv - Sq : 0; }
grid::StreamPlan stream_plan_for(long long bh, int Sq, int off) {
  return grid::stream_plan(bh, Sq, kStreamBM, kStreamMaxGroups, kStreamMinUnits, kStreamPieceCost, off);
}
bool split_applies(long long bh, int Sq, bool causal, const KvSpec& kv) {
  if (!causal || kv.window > 0 || kv.mask || paired_grid(bh, Sq)) return false;
  // Against a long cache every query tile does about the same work, so the
  // key-group grid is balanced once it has a workgroup per CU (a chunk of 512
  // after 4096 cached tokens, 64 heads: 80 us there against 83 us stream-K);
  // below that stream-K wins (8 heads, 2048 after 6144 cached: 1.21x).
  if (kv.lens && (kv.max_kv < Sq || bh * ((Sq + 127) / 128) >= grid::kCUs)) return false;
  const int nqt = (Sq + kStreamBM - 1) / kStreamBM;
  if (nqt > kStreamMaxTiles || bh * nqt > kSplitCounters) return false;
  const grid::StreamPlan p = stream_plan_for(bh, Sq, stream_off(Sq, kv));
  return p.ok && p.units >= (long long)kStreamMinShare * kStreamMaxGroups;
}
// The plan's tables for the last shape seen on this thread (serving loops
// repeat shapes; the ranges come from a search over the greedy cover).
SplitArgs stream_tables_cached(long long bh, int Sq, int off, const grid::StreamPlan& p) {
  const long long key[3] = {bh, Sq, off};
  thread_local long long last[3] = {-1, -1, -1};
  thread_local SplitArgs tab;
  if (!std::equal(key, key + 3, last)) {
    const grid::StreamRanges r = grid::stream_ranges(p, bh, Sq, kStreamBM, kStreamMergeCost, off);
    tab = SplitArgs{};
    tab.per = p.per;
    for (int j = 0, s = 0; j <= p.nqt; j++) {
      tab.tstart[j] = s;
      if (j < p.nqt) s += grid::stream_ntiles(Sq, grid::stream_pair_qt(j, p.nqt), kStreamBM, off);
    }
    for (int w = 0; w <= p.G; w++) tab.wstart[w] = r.wstart[w];
    for (int w = 0; w < p.G; w++) {
      tab.wtile[w] = (uint16_t)r.first_tile[w];
      tab.wlo[w] = (uint8_t)r.lo_owner[w];
      tab.whi[w] = (uint8_t)r.hi_owner[w];
    }
    std::copy(key, key + 3, last);
  }
  return tab;
}
size_t split_workspace_bytes(long long bh, int Sq, int D, const KvSpec& kv) {
  const grid::StreamPlan p = stream_plan_for(bh, Sq, stream_off(Sq, kv));
  // per slot: BM x D fp16 values, then BM x 4 floats
  return kSplitCounterBytes + 2 * (size_t)p.G * kStreamBM * (sizeof(uint16_t) * (size_t)D + 4 * sizeof(float));
}
}  // namespace

size_t prefill_split_workspace_bytes(int B, int Sq, int Hq, int D, bool causal) {
  const long long bh = (long long)B * Hq;
  const KvSpec kv{};
  return split_applies(bh, Sq, causal, kv) ? split_workspace_bytes(bh, Sq, D, kv) : 0;
}

size_t prefill_cache_split_workspace_bytes(int B, int Sq, int Hq, int D, int max_kv, bool causal, int window) {
  const long long bh = (long long)B * Hq;
  static const int32_t probe = 0;  // stands for the per-sequence lengths: only its presence matters here
  KvSpec kv{};
  kv.lens = &probe;
  kv.max_kv = max_kv;
  kv.window = window;
  return split_applies(bh, Sq, causal, kv) ? split_workspace_bytes(bh, Sq, D, kv) : 0;
}

hipError_t launch_prefill_bf16_split(const void* q, const void* k, const void* v, void* out, int B, int Sq, int Hq,
                                     int Hkv, int D, bool causal, float scale, const KvSpec& kv, void* ws,
                                     hipStream_t st) {
  const long long bh = (long long)B * Hq;
  if (!ws || !split_applies(bh, Sq, causal, kv))
    return launch_prefill_bf16(q, k, v, out, B, Sq, Hq, Hkv, D, causal, scale, kv, nullptr, st);
  const float c_log2 = (float)((double)scale * 1.4426950408889634);
  const int off = stream_off(Sq, kv);
  const grid::StreamPlan p = stream_plan_for(bh, Sq, off);
  const size_t nslots = 2 * (size_t)p.G;
  SplitArgs sa = stream_tables_cached(bh, Sq, off, p);
  sa.cnt = reinterpret_cast<int*>(ws);
  sa.o = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + kSplitCounterBytes);
  sa.ml = reinterpret_cast<float*>(sa.o + nslots * kStreamBM * D / 2);
  const dim3 grid((unsigned)p.G), block(512);
#define RCGQA_SPLIT_LAUNCH(DD, GG)                                                                                   \
  hipLaunchKernelGGL((prefill_bf16_kernel<DD, 8, GG, 1, 64, false, true>), grid, block, 0, st, (const bf16*)q,     \
                     (const bf16*)k, (const bf16*)v, (bf16*)out, Sq, Hq, Hkv, 1, c_log2, p.nqt, p.nqt, kv, nullptr, sa)
  if (kv.lens) {
    if (D == 64) RCGQA_SPLIT_LAUNCH(64, true);
    else RCGQA_SPLIT_LAUNCH(128, true);
  } else {
    if (D == 64) RCGQA_SPLIT_LAUNCH(64, false);
    else RCGQA_SPLIT_LAUNCH(128, false);
  }
#undef RCGQA_SPLIT_LAUNCH
  return hipGetLastError();
}

namespace {
// The choice for the last shape seen on this thread is kept: serving loops
// repeat shapes, and the estimate walks every workgroup of both grids.
grid::KeyGroupGrid key_group_grid_cached(long long bh, int Sq, bool causal, const KvSpec& kv) {
  const long long nk = kv.lens ? kv.max_kv : Sq;
  const long long key[5] = {bh, Sq, causal, kv.lens ? kv.max_kv : -1, kv.window};
  thread_local long long last[5] = {-1, -1, -1, -1, -1};
  thread_local grid::KeyGroupGrid last_choice{false, 0};
  if (!std::equal(key, key + 5, last)) {
    last_choice = grid::key_group_grid(bh, Sq, causal, nk, kv.window);
    std::copy(key, key + 5, last);
  }
  return last_choice;
}
}  // namespace

hipError_t launch_prefill_bf16(const void* q, const void* k, const void* v, void* out, int B, int Sq, int Hq,
                               int Hkv, int D, bool causal, float scale, const KvSpec& kv, const float* q_rope,
                               hipStream_t st) {
  const float c_log2 = (float)((double)scale * 1.4426950408889634);
  // Every K/V tile brought into LDS serves the workgroup's query rows, so 8
  // waves (256 rows) halve the tile traffic per flop against 4 waves (128
  // rows).  Both run 8 waves per CU (one 8-wave or two 4-wave workgroups).
  // Causal grids pair heavy and light query tiles so all workgroups do equal
  // work.  In order of preference: 8 waves when that paired grid still has
  // 512 workgroups or more; 4 waves when their grid (paired if that keeps 512
  // workgroups) has 512 or more; otherwise one 8-wave workgroup per CU in
  // several key groups, 128-row tiles in two groups or 64-row tiles in four,
  // whichever is estimated to finish first.
  const long long bh = (long long)B * Hq;
  const int nqt8 = (Sq + 255) / 256, nqt4 = (Sq + 127) / 128;
  // Under a sliding window a block of R query rows walks about window + R
  // keys where each row sees window keys, so windows shorter than 2048 keys
  // take 128-row tiles (window 256: 104 -> 86 us, 1024: 170 -> 164 us on
  // B=2 S=4096 Hq=Hkv=32 D=128).
  const bool short_window = kv.window > 0 && kv.window < 2048;
  // the 8-wave grid stages mask tiles in LDS with 16-byte loads: rows of a multiple of 8 entries
  const bool mask_ok = !kv.mask || (kv.msr % 8 == 0 && kv.msr >= 8);
  // With D = 64 a K/V tile is half the bytes, and the 4-wave grid measured as
  // fast or faster (interleaved, bit-identical: B=2 S=4096 Hq=32 +2%, B=1
  // S=4096 Hq=32 Hkv=8 +0.3%, B=4 S=2048 Hq=32 +5%, B=1 S=8192 Hq=16 +0.3%);
  // with D = 128 it is 4% slower on the same shapes.
  if (D == 128 && causal && nqt8 > 1 && bh * ((nqt8 + 1) / 2) >= 512 && !short_window && mask_ok) {
    launch_nw<8, 1>(q, k, v, out, B, Sq, Hq, Hkv, D, causal, c_log2, (nqt8 + 1) / 2, kv, q_rope, st);
  } else {
    const bool pair4 = causal && nqt4 > 1 && bh * ((nqt4 + 1) / 2) >= 512;
    const int npairs = pair4 ? (nqt4 + 1) / 2 : nqt4;
    if (bh * npairs >= 512) {
      launch_nw<4, 1>(q, k, v, out, B, Sq, Hq, Hkv, D, causal, c_log2, npairs, kv, q_rope, st);
    } else {
      const grid::KeyGroupGrid g = key_group_grid_cached(bh, Sq, causal, kv);
      if (g.four)
        launch_nw<8, 4, 32>(q, k, v, out, B, Sq, Hq, Hkv, D, causal, c_log2, g.npairs, kv, q_rope, st);
      else
        launch_nw<8, 2>(q, k, v, out, B, Sq, Hq, Hkv, D, causal, c_log2, g.npairs, kv, q_rope, st);
    }
  }
  return hipGetLastError();
}

}  // namespace rcgqa
