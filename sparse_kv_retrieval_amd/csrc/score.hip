// Score + threshold over every compressed entry, and the gathered re-scoring
// that feeds the native top-k.
//
// The full scan implements the lookahead index score and its loading rule
// ([BLOG] §3.1 of the FlashMemory-DeepSeek-V4 write-up: I = sigma(sum_j w_j
// ReLU(q_j . K_s)), entries with I >= 0.5 are loaded). It is the O(B*L*N)
// stream over the keys and is bound by HBM bandwidth. Each wave owns a
// contiguous range of 64-entry mask words, so it reloads its query only
// when it crosses into another (layer, sequence). Each word is two 32-entry
// MFMA tiles, and the wave ballot of the two tiles' selections is the 64-bit
// mask word.
#include <algorithm>

#include "kernels.hpp"
#include "scorer.hpp"
#include "cursor.hpp"

namespace lsa {

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt in 6:4, lgkmcnt in 11:8).
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
template <int STEP>
__device__ __forceinline__ void vm_wait_pending(int pending) {
  // Vector-memory loads complete in issue order, so "at most STEP*pending
  // outstanding" means every tile older than the last `pending` tiles has
  // landed in LDS.
  switch (pending) {
    case 0: vm_wait<0>(); break;
    case 1: vm_wait<STEP>(); break;
    case 2: vm_wait<2 * STEP>(); break;
    default: vm_wait<3 * STEP>(); break;
  }
  asm volatile("" ::: "memory");
}

#define LSA_AS3(p) ((__attribute__((address_space(3))) void*)(p))

// Block barrier for LDS traffic only. __syncthreads() also fences global memory,
// so it waits for every outstanding vector load (vmcnt(0)), and that would drain
// the key DMAs still in flight. Here the LDS operations of this wave
// (lgkmcnt) complete first, and the barrier is then the bare s_barrier. The
// DMAs that a tile depends on are waited for explicitly with vm_wait_pending.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt at their maxima (no wait)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Score + select: keys streamed HBM -> registers -> LDS -> MFMA, two waves per tile.
//
// A block is one pair of waves and owns a contiguous run of mask words. Each
// word is two 32-entry tiles. Wave h loads half of every tile with coalesced
// 16-byte vector loads (each load instruction covers 1 KiB of contiguous key
// rows) and keeps D tiles in flight in registers. When a tile's turn comes, it
// writes the tile into one of two LDS stages. fp8 keys are widened to bf16 on
// the way (exact, one conversion instruction per two values), so both waves
// then run the bf16 MFMA on the same operands. The LDS layout (lds_chunk)
// swizzles 16-byte chunks so that the stores and the operand reads (lane n
// reads row n) are free of bank conflicts.
//
// Wave h scores heads [32h, 32h+32). Wave 1 passes its gate/ReLU partial sums
// to wave 0 through LDS, and wave 0 finishes tile j-1 (threshold, ballot,
// mask word, optional sigmoid) in iteration j. There is one barrier per tile.
// After it, tile j is complete in LDS, the previous partial is visible, and
// the stage written next iteration is no longer being read.
template <int KT, int DH>
struct TileIO {
  static constexpr int GESZ = KT == KEY_F32 ? 4 : (KT == KEY_BF16 ? 2 : 1);  // stored element
  static constexpr int LESZ = KT == KEY_F32 ? 4 : 2;                         // element in LDS
  static constexpr int GRB = DH * GESZ;      // stored row bytes
  static constexpr int LRB = DH * LESZ;      // LDS row bytes
  static constexpr int GSUB = 32 * GRB;      // stored tile bytes
  static constexpr int LSUB = 32 * LRB;      // LDS tile bytes
  static constexpr int NLI = GSUB / 1024;    // 1 KiB load instructions per tile (>= 1)
  static constexpr int NLW = NLI >= 2 ? NLI / 2 : 1;  // per wave
  static constexpr int GCPR = GRB / 16;      // stored 16-byte chunks per row
  static constexpr int LCPR = LRB / 16;      // LDS 16-byte chunks per row
  // fp8 rows of 8+ stored chunks: one 8-lane write group covers one row
  static constexpr bool ROT = KT == KEY_FP8 && GCPR >= 8;
};

// Where a scored tile's results go: entry n of the tile is row `row` (valid
// if the entry exists), in mask word `word` of layer `l`.
struct TileMeta {
  bool valid = false;
  int64_t row = 0;
  uint64_t* mw = nullptr;  // the tile's mask word
  float* so = nullptr;     // the layer's sigmoid scores, or null
  float scale = 1.0f;      // fp8 keys: the entry's scale
};

// Threshold, ballot and stores of one tile, given its full logit x (lane n of
// both lane groups holds entry n). Tiles come in pairs per 64-bit mask word:
// the even tile's ballot waits in bits0 for the odd one.
__device__ __forceinline__ void finish_tile(const ScoreArgs& a, const TileMeta& m, float x, int odd,
                                            uint32_t& bits0, int lane, int g) {
  const uint32_t bits = (uint32_t)__ballot(m.valid && x >= a.thr);
  if (m.so != nullptr && g == 0 && m.valid) m.so[m.row] = 1.0f / (1.0f + __expf(-x));
  if (odd) {
    if (lane == 0) *m.mw = (uint64_t)bits0 | ((uint64_t)bits << 32);
  } else {
    bits0 = bits;
  }
}

template <int KT, int DH, int D>
__global__ __launch_bounds__(128) void score_select_kernel(const ScoreArgs a) {
  using IO = TileIO<KT, DH>;
  using S_t = Scorer<KT == KEY_F32 ? KEY_F32 : KEY_BF16, DH, 1, TileIO<KT, DH>::ROT>;
  static_assert(S_t::ROW_BYTES == IO::LRB, "LDS row layout");
  __shared__ __attribute__((aligned(16))) char stage[2][IO::LSUB];
  __shared__ float xpart[2][32];

  const int lane = threadIdx.x & 63, g = lane >> 5, n = lane & 31;
  const int h = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // which half of the heads
  const SeqTab t(a.key_off, a.mwo);
  // Pairs form groups of G. A group owns a contiguous run of mask words, and
  // its pairs take every G-th word of the run. The G pairs then stream
  // neighbouring tiles, which keeps DRAM accesses local, while each pair stays
  // inside one (layer, sequence) for long stretches.
  const int G = a.group;
  const int64_t ng = gridDim.x / G;
  const int64_t grp = blockIdx.x / G, off = blockIdx.x % G;
  const int64_t gbeg = grp * a.total_words / ng;
  const int64_t gend = (grp + 1) * a.total_words / ng;
  const int64_t nwords = gend - gbeg > off ? (gend - gbeg - off + G - 1) / G : 0;
  const int J = (int)(2 * nwords);  // tiles of this pair
  if (J == 0) return;

  // This wave's load instructions: [i0, i0 + NLW), or none for 1 KiB tiles on wave 1.
  const int i0 = IO::NLI >= 2 ? h * IO::NLW : 0;
  const bool loads = IO::NLI >= 2 || h == 0;
  // per instruction: row within the tile, and the stored chunk of that row
  int lrow[IO::NLW], lchunk[IO::NLW];
  uint32_t loff[IO::NLW];  // byte offset within the tile (out of range: this wave loads nothing)
#pragma unroll
  for (int i = 0; i < IO::NLW; ++i) {
    const int p = (i0 + i) * 1024 + lane * 16;
    lrow[i] = p / IO::GRB;
    lchunk[i] = (p % IO::GRB) / 16;
    loff[i] = loads ? (uint32_t)p : BUF_OOB;
  }

  u32x4 R[D][IO::NLW];
  float SC[D];
  WordCursor ic, cc;
  ic.place(a, t, gbeg + off);
  cc = ic;

  S_t S;
  int cur_l = -1, cur_b = -1;
  f32x16 acc[1];        // MFMA result of the last tile issued
  TileMeta m1, m2;      // tiles j-1 and j-2 (wave 0 finishes them)
  float p2 = 0.0f;      // wave 0's half of the head sum of tile j-2
  uint32_t bits0 = 0;

  // Loads of tile JJ into register slot SLOT. Every slot issues the same
  // loads whether or not it is LIVE (a tile of this pair). The buffer
  // resource covers exactly the tile's existing rows (none for a dead slot),
  // so the rows past a sequence's end read as zeros. With the resource based
  // at the tile, each lane's offsets are constants.
#define LSA_LOAD_TILE(SLOT, JJ, LIVE)                                                                 \
  do {                                                                                              \
    const bool live_ = (LIVE);                                                                      \
    const int32_t e_ = ic.e0 + ((JJ) & 1) * 32;                                                     \
    const int64_t row_ = ic.row0 + e_;                                                              \
    const uint32_t nr_ = live_ ? (uint32_t)uni(max(0, min(32, ic.nb - e_))) : 0u;                     \
    const auto rk_ = buf_rsrc(ic.keys + row_ * IO::GRB, nr_ * IO::GRB);                             \
    _Pragma("unroll") for (int i = 0; i < IO::NLW; ++i) R[SLOT][i] = buf_load16_nt(rk_, loff[i]);   \
    if constexpr (KT == KEY_FP8) {                                                                  \
      const auto rs_ = buf_rsrc(ic.scale + row_, nr_ * 4);                                          \
      SC[SLOT] = __uint_as_float(buf_load4(rs_, n * 4));                                            \
    }                                                                                               \
    if (live_ && ((JJ) & 1)) ic.advance(a, t, G);                                                   \
  } while (0)

  // The prologue keeps its slots in issue order (the sched barrier), so slot
  // s is always the oldest load group when tile s is written.
#pragma unroll
  for (int s = 0; s < D; ++s) {
    LSA_LOAD_TILE(s, s, s < J);
    __builtin_amdgcn_sched_barrier(0);
  }

  // The loop runs whole groups of D slots. A slot past the last tile (j >= J)
  // only issues its (out-of-range) refill. With no early exit, every path
  // around the loop issues the same loads, so the compiler's wait before
  // writing tile j covers tile j's loads only, and the D - 1 younger tiles
  // stay in flight.
  const int NIT = (J + D - 1) / D;
  for (int it = 0; it < NIT; ++it) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      const int j = it * D + s;
      const bool live = j < J;
      char* st = &stage[j & 1][0];
      // write this wave's half of tile j into LDS (waits for its loads)
      if (live && loads) {
#pragma unroll
        for (int i = 0; i < IO::NLW; ++i) {
          const int r = lrow[i];
          char* rowp = st + r * IO::LRB;
          if constexpr (KT == KEY_FP8) {
            const u32x4 v = R[s][i];
            const u32x2 b0 = e4m3x4_to_bf16x4(v[0]), b1 = e4m3x4_to_bf16x4(v[1]);
            const u32x2 b2 = e4m3x4_to_bf16x4(v[2]), b3 = e4m3x4_to_bf16x4(v[3]);
            const int c0 = 2 * lchunk[i], c1 = c0 + 1;
            *(u32x4*)(rowp + lds_chunk<IO::LCPR, IO::ROT>(c0, r) * 16) = u32x4{b0[0], b0[1], b1[0], b1[1]};
            *(u32x4*)(rowp + lds_chunk<IO::LCPR, IO::ROT>(c1, r) * 16) = u32x4{b2[0], b2[1], b3[0], b3[1]};
          } else {
            *(u32x4*)(rowp + lds_chunk<IO::LCPR, IO::ROT>(lchunk[i], r) * 16) = R[s][i];
          }
        }
      }
      float scale = 1.0f;
      if constexpr (KT == KEY_FP8) scale = SC[s];
      // refill this slot with tile j + D
      LSA_LOAD_TILE(s, j + D, j + D < J);
      if (!live) continue;
      // Tile j's MFMAs are issued at the end of iteration j. Their result is
      // consumed one iteration later (gate/ReLU partial of tile j-1, below),
      // so the MFMA chain runs while this wave writes and loads the next
      // tile. Wave 0 finishes a tile one iteration after that, once wave 1's
      // half of the head sum is in LDS.
      lds_barrier();  // tile j complete in LDS; wave 1's partial of tile j-2 visible
      S.read_keys_lds(st);
      // keep the partial below the barrier and the operand reads: it is what
      // waits for tile j-1's MFMA chain
      __builtin_amdgcn_sched_barrier(0);
      if (j > 0) {
        float p = S.partial(acc);
        p = sum_halves(p);
        if constexpr (KT == KEY_FP8) p *= m1.scale;
        if (h == 1) {
          if (g == 0) xpart[(j - 1) & 1][n] = p;
        } else {
          if (j > 1) finish_tile(a, m2, p2 + xpart[(j - 2) & 1][n], (j - 2) & 1, bits0, lane, g);
          p2 = p;
          m2 = m1;
        }
      }
      if (cc.l != cur_l || cc.b != cur_b) {
        S.load_query(a.q[cc.l], a.w[cc.l], cc.b, a.n_h, 32 * h);
        cur_l = cc.l;
        cur_b = cc.b;
      }
      {
        const int32_t se = cc.e0 + (j & 1) * 32 + n;
        m1.valid = se < cc.nb;
        m1.row = cc.row0 + se;
        m1.mw = cc.mask + cc.word;
        m1.so = cc.score;
        m1.scale = scale;
      }
      S.mma(acc);
      if (j & 1) cc.advance(a, t, G);
    }
  }
#undef LSA_LOAD_TILE
  // drain: tile J-2 (partial already taken) and tile J-1 (MFMAs in flight)
  lds_barrier();
  {
    float p = S.partial(acc);
    p = sum_halves(p);
    if constexpr (KT == KEY_FP8) p *= m1.scale;
    if (h == 1) {
      if (g == 0) xpart[(J - 1) & 1][n] = p;
    } else {
      if (J > 1) finish_tile(a, m2, p2 + xpart[(J - 2) & 1][n], (J - 2) & 1, bits0, lane, g);
      p2 = p;
    }
  }
  lds_barrier();
  if (h == 0) finish_tile(a, m1, p2 + xpart[(J - 1) & 1][n], (J - 1) & 1, bits0, lane, g);
}

// Gathered scoring for the top-k: y = sum_j w'_j ReLU(q'_j . K_s) for each s in
// the union list ([BLOG] §3.2: the native indexer works only inside the loaded
// subset).
//
// The 32-entry tiles of all (layer, sequence) lists are numbered
// consecutively, and each pair of waves takes a contiguous run of them. The
// pipeline is the one of score_select: register-staged loads D tiles ahead,
// a double-buffered swizzled LDS stage, 32 heads per wave, and one barrier per
// tile. The key rows are gathered through the index list. A load instruction
// covers four whole 256-byte rows, so every row is fetched fully coalesced.
// Each tile's indices are loaded D tiles before its keys. The key loads then
// never wait on a load issued after the older loads still in flight.
struct TileCursor {
  int l, b;
  int32_t jt, nt;     // tile within sequence b, tiles of sequence b
  int64_t base;       // first row of sequence b (also where its list starts)
  int32_t cnt;        // entries in b's list
  int32_t nrow;       // rows of sequence b
  int32_t rbase;      // contiguous mode: first packed row of sequence b's list
  const char* keys;   // layer l's keys and fp8 scales (past the last layer: the last layer's, unused)
  const float* scale;
  template <bool CONTIG>
  __device__ __forceinline__ void load_layer(const TopkScoreArgs& a) {
    const int ll = l < a.L ? l : a.L - 1;
    keys = (const char*)(CONTIG ? a.sub_keys[ll] : a.keys[ll]);
    scale = a.scale[ll];
  }
  __device__ __forceinline__ void load_seq(const TopkScoreArgs& a, const int32_t* tp, const int32_t* rp) {
    nt = uni(tp[b + 1]) - uni(tp[b]);
    base = uni(a.key_off[b]);
    nrow = (int32_t)(uni(a.key_off[b + 1]) - base);
    cnt = uni(a.count[b]);
    rbase = rp ? uni(rp[b]) : 0;
  }
  template <bool CONTIG>
  __device__ __forceinline__ void place(const TopkScoreArgs& a, const int32_t* tp, const int32_t* rp, int64_t t) {
    const int64_t tpl = uni(tp[a.B]);
    l = uni((int32_t)(t / tpl));
    const int32_t tt = (int32_t)(t - (int64_t)l * tpl);
    b = uni(upper_seq(tp, a.B, tt));
    jt = tt - uni(tp[b]);
    load_seq(a, tp, rp);
    load_layer<CONTIG>(a);
  }
  template <bool CONTIG>
  __device__ __forceinline__ void next(const TopkScoreArgs& a, const int32_t* tp, const int32_t* rp) {
    if (++jt < nt) return;
    jt = 0;
    do {
      if (++b == a.B) {
        b = 0;
        ++l;
        load_layer<CONTIG>(a);
      }
    } while (uni(tp[b + 1]) == uni(tp[b]));
    load_seq(a, tp, rp);
  }
};

// CONTIG: the keys of the lists are packed in list order in sub_keys (list
// entry i of sequence b is row rp[b] + i), so every tile is 32 consecutive
// rows and no index load precedes the key loads (fp8 scales are still read
// through the list from the full scale array). Used for the per-step top-k
// over the resident subset. At most TOPK_CONTIG_MAX_B sequences.
#if LSA_DEBUG_CHECKS
static __device__ unsigned int g_topk_range_errors;
__device__ __forceinline__ void range_error() { atomicAdd(&g_topk_range_errors, 1u); }
#else
__device__ __forceinline__ void range_error() {}
#endif

hipError_t topk_take_range_errors(unsigned int* out) {
#if LSA_DEBUG_CHECKS
  hipError_t e = hipMemcpyFromSymbol(out, HIP_SYMBOL(g_topk_range_errors), sizeof(unsigned int));
  if (e != hipSuccess) return e;
  const unsigned int zero = 0;
  return hipMemcpyToSymbol(HIP_SYMBOL(g_topk_range_errors), &zero, sizeof(unsigned int));
#else
  *out = 0;
  return hipSuccess;
#endif
}

template <int KT, int DH, int D, bool CONTIG>
__global__ __launch_bounds__(128) void topk_score_kernel(const TopkScoreArgs a) {
  using IO = TileIO<KT, DH>;
  using S_t = Scorer<KT == KEY_F32 ? KEY_F32 : KEY_BF16, DH, 1, TileIO<KT, DH>::ROT>;
  static_assert(IO::GRB == 16 * (IO::GRB / 16), "row size");
  constexpr int MAXB = CONTIG ? TOPK_CONTIG_MAX_B : LSA_TOPK_MAX_B;
  __shared__ __attribute__((aligned(16))) char stage[2][IO::LSUB];
  __shared__ float xpart[2][32];
  __shared__ int32_t tp[MAXB + 1];
  __shared__ int32_t rps[CONTIG ? MAXB + 1 : 1];
  // this block's counts for the histogram of one (layer, sequence): two 16-bit bins per word
  __shared__ uint32_t lh[TOPK_BINS / 2];
  const int32_t* rp = CONTIG ? rps : nullptr;
  for (int i = threadIdx.x; i < TOPK_BINS / 2; i += blockDim.x) lh[i] = 0u;

  const int lane = threadIdx.x & 63, g = lane >> 5, n = lane & 31;
  const int h = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if constexpr (CONTIG) block_list_prefix(a.count, a.B, tp, rps);
  else block_tile_prefix(a.count, a.B, tp);
  const int64_t total = (int64_t)tp[a.B] * a.L;
  const int64_t np = gridDim.x;
  const int64_t t0 = (int64_t)blockIdx.x * total / np;
  const int64_t t1 = ((int64_t)blockIdx.x + 1) * total / np;
  const int J = (int)(t1 - t0);
  if (J == 0) return;

  const int i0 = IO::NLI >= 2 ? h * IO::NLW : 0;
  const bool loads = IO::NLI >= 2 || h == 0;
  int lrow[IO::NLW], lchunk[IO::NLW];
#pragma unroll
  for (int i = 0; i < IO::NLW; ++i) {
    const int p = (i0 + i) * 1024 + lane * 16;
    lrow[i] = p / IO::GRB;
    lchunk[i] = (p % IO::GRB) / 16;
  }

  u32x4 R[D][IO::NLW];
  float SC[D];
  int32_t IX[2 * D][IO::NLW];  // list entries of the rows this lane loads, 2D tiles deep
  int32_t IXS[2 * D];          // (fp8) list entry of row n, for the scale
  TileCursor xc, ic, cc;       // index, key and compute cursors
  xc.place<CONTIG>(a, tp, rp, t0);
  ic = xc;
  cc = xc;

  // As in score_select, every slot issues its loads whether or not it is LIVE:
  // a dead slot, or a list entry past the end of a list, reads out of range
  // and gets zeros (list entry 0: row 0 of the sequence, whose score is
  // dropped).
#define LSA_LOAD_IDX(SLOT, LIVE)                                                                \
  do {                                                                                         \
    const bool live_ = (LIVE);                                                                 \
    const uint32_t e_ = (uint32_t)xc.jt * 32;                                                  \
    const auto ri_ = buf_rsrc(a.idx + xc.base, (uint32_t)xc.cnt * 4);                          \
    if constexpr (!CONTIG) {                                                                   \
      _Pragma("unroll") for (int i = 0; i < IO::NLW; ++i)                                      \
        IX[SLOT][i] = (int32_t)buf_load4(ri_, live_ ? (e_ + lrow[i]) * 4 : BUF_OOB);           \
    }                                                                                          \
    if constexpr (KT == KEY_FP8) IXS[SLOT] = (int32_t)buf_load4(ri_, live_ ? (e_ + n) * 4 : BUF_OOB); \
    if (live_) xc.next<CONTIG>(a, tp, rp);                                                     \
  } while (0)
#define LSA_LOAD_KEYS(SLOT, XSLOT, LIVE)                                                       \
  do {                                                                                         \
    const bool live_ = (LIVE);                                                                 \
    if constexpr (CONTIG) {                                                                    \
      const auto rk_ = buf_rsrc(ic.keys + (int64_t)ic.rbase * IO::GRB, (uint32_t)ic.cnt * IO::GRB); \
      const uint32_t e_ = (uint32_t)ic.jt * 32;                                                \
      _Pragma("unroll") for (int i = 0; i < IO::NLW; ++i)                                      \
        R[SLOT][i] = buf_load16_nt(                                                            \
            rk_, live_ && loads ? (e_ + lrow[i]) * IO::GRB + lchunk[i] * 16 : BUF_OOB);        \
    } else {                                                                                   \
      const auto rk_ = buf_rsrc(ic.keys + ic.base * IO::GRB, (uint32_t)ic.nrow * IO::GRB);     \
      _Pragma("unroll") for (int i = 0; i < IO::NLW; ++i) {                                    \
        const bool in_ = LSA_DEBUG_CHECKS == 0 || (uint32_t)IX[XSLOT][i] < (uint32_t)ic.nrow;    \
        if (LSA_DEBUG_CHECKS && live_ && loads && !in_) range_error();                         \
        R[SLOT][i] = buf_load16_nt(                                                            \
            rk_, live_ && loads && in_ ? (uint32_t)IX[XSLOT][i] * IO::GRB + lchunk[i] * 16 : BUF_OOB); \
      }                                                                                        \
    }                                                                                          \
    if constexpr (KT == KEY_FP8) {                                                             \
      const auto rs_ = buf_rsrc(ic.scale + ic.base, (uint32_t)ic.nrow * 4);                    \
      const bool ins_ = LSA_DEBUG_CHECKS == 0 || (uint32_t)IXS[XSLOT] < (uint32_t)ic.nrow;     \
      if (LSA_DEBUG_CHECKS && live_ && !ins_) range_error();                                   \
      SC[SLOT] = __uint_as_float(buf_load4(rs_, live_ && ins_ ? (uint32_t)IXS[XSLOT] * 4 : BUF_OOB)); \
    }                                                                                          \
    if (live_) ic.next<CONTIG>(a, tp, rp);                                                     \
  } while (0)

  // prologue: indices for tiles 0 .. 2D-1 and keys for tiles 0 .. D-1, issued
  // in the order of the steady state (keys of tile s, then indices of tile
  // s + D), so the waits in the loop are the same for every slot
#pragma unroll
  for (int s = 0; s < D; ++s) {
    LSA_LOAD_IDX(s, s < J);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int s = 0; s < D; ++s) {
    LSA_LOAD_KEYS(s, s, s < J);
    LSA_LOAD_IDX(D + s, D + s < J);
    __builtin_amdgcn_sched_barrier(0);
  }

  S_t S;
  int cur_l = -1, cur_b = -1;
  float pprev = 0.0f;
  bool vprev = false;
  int64_t oprev = 0;
  int64_t hprev = 0;  // histogram of the previous tile's (layer, sequence)
  // Wave 0 writes every score and counts it in lh, the block's histogram of the current
  // (layer, sequence) hcur. The counts go to the global histogram (non-zero bins, one
  // atomic each) when the (layer, sequence) changes, before a 16-bit count could
  // overflow, and at the end: far fewer global atomics than one per score, which would
  // serialise on the few bins that hold most scores.
  int64_t hcur = -1;
  uint32_t since = 0;  // scores counted in lh since its last flush (at most 65535 per bin)
  auto flush = [&]() {
    if (hcur >= 0 && a.hist) {
      for (int i = lane; i < TOPK_BINS / 2; i += 64) {
        const uint32_t v = lh[i];
        if (v) {
          if (v & 0xFFFFu) atomicAdd(a.hist + hcur + 2 * i, v & 0xFFFFu);
          if (v >> 16) atomicAdd(a.hist + hcur + 2 * i + 1, v >> 16);
          lh[i] = 0u;
        }
      }
    }
    since = 0;
  };
  // wave 0, every lane: the score of list position o when `on`, in (layer, sequence) hb
  auto put = [&](bool on, int64_t o, int64_t hb, float y) {
    if (hb != hcur || since > 65535u - 64u) {  // uniform
      flush();
      hcur = hb;
    }
    since += (uint32_t)__popcll(__ballot(on));
    if (on) {
      a.ys[o] = y;
      if (a.hist) {
        const uint32_t bin = order_key(y) >> (32 - TOPK_HBITS);
        atomicAdd(&lh[bin >> 1], 1u << (16 * (bin & 1)));
      }
    }
  };

  // Whole groups of 2D slots, no early exit (see score_select): a slot past the
  // last tile only issues its out-of-range refills.
  const int NIT = (J + 2 * D - 1) / (2 * D);
  for (int it = 0; it < NIT; ++it) {
#pragma unroll
    for (int s = 0; s < 2 * D; ++s) {
      const int j = it * 2 * D + s;
      const bool live = j < J;
      const int rs = s % D;  // register slot of tile j
      char* st = &stage[j & 1][0];
      if (live && loads) {
#pragma unroll
        for (int i = 0; i < IO::NLW; ++i) {
          const int r = lrow[i];
          char* rowp = st + r * IO::LRB;
          if constexpr (KT == KEY_FP8) {
            const u32x4 v = R[rs][i];
            const u32x2 b0 = e4m3x4_to_bf16x4(v[0]), b1 = e4m3x4_to_bf16x4(v[1]);
            const u32x2 b2 = e4m3x4_to_bf16x4(v[2]), b3 = e4m3x4_to_bf16x4(v[3]);
            const int c0 = 2 * lchunk[i], c1 = c0 + 1;
            *(u32x4*)(rowp + lds_chunk<IO::LCPR, IO::ROT>(c0, r) * 16) = u32x4{b0[0], b0[1], b1[0], b1[1]};
            *(u32x4*)(rowp + lds_chunk<IO::LCPR, IO::ROT>(c1, r) * 16) = u32x4{b2[0], b2[1], b3[0], b3[1]};
          } else {
            *(u32x4*)(rowp + lds_chunk<IO::LCPR, IO::ROT>(lchunk[i], r) * 16) = R[rs][i];
          }
        }
      }
      float scale = 1.0f;
      if constexpr (KT == KEY_FP8) scale = SC[rs];
      LSA_LOAD_KEYS(rs, (s + D) % (2 * D), j + D < J);
      LSA_LOAD_IDX(s, j + 2 * D < J);
      if (!live) continue;
      lds_barrier();
      S.read_keys_lds(st);
      if (h == 0 && j > 0) {
        const float y = pprev + xpart[(j - 1) & 1][n];
        put(g == 0 && vprev, oprev, hprev, y);
      }
      if (cc.l != cur_l || cc.b != cur_b) {
        S.load_query(a.q[cc.l], a.w[cc.l], cc.b, a.n_h, 32 * h);
        cur_l = cc.l;
        cur_b = cc.b;
      }
      f32x16 acc[1];
      S.mma(acc);
      float p = S.partial(acc);
      p = sum_halves(p);
      if constexpr (KT == KEY_FP8) p *= scale;
      const int32_t e = cc.jt * 32 + n;
      if (h == 1) {
        if (g == 0) xpart[j & 1][n] = p;
      } else {
        pprev = p;
        vprev = e < cc.cnt;
        oprev = (int64_t)cc.l * a.rows_total + cc.base + e;
        hprev = ((int64_t)cc.l * a.B + cc.b) * TOPK_BINS;
      }
      cc.next<CONTIG>(a, tp, rp);
    }
  }
#undef LSA_LOAD_IDX
#undef LSA_LOAD_KEYS
  lds_barrier();
  if (h == 0) {
    const float y = pprev + xpart[(J - 1) & 1][n];
    put(g == 0 && vprev, oprev, hprev, y);
    flush();
  }
}

__global__ void topk_hist_zero_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = 0u;
}

hipError_t launch_topk_hist_zero(uint32_t* hist, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(topk_hist_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st, hist, n);
  return hipGetLastError();
}

// ------------------------------------------------------------------ launch
// Tiles in flight per wave (D). The default keeps about 16 KiB of key loads in
// flight per wave pair; `depth` > 0 overrides it for d_h = 128.
template <int KT, int DH, int D>
static hipError_t launch_score_d(const ScoreArgs& a, int pairs, hipStream_t st) {
  hipLaunchKernelGGL((score_select_kernel<KT, DH, D>), dim3(pairs), dim3(128), 0, st, a);
  return hipGetLastError();
}
template <int KT, int DH>
static hipError_t launch_score_t(const ScoreArgs& a, int pairs, int depth, hipStream_t st) {
  constexpr int DDEF = TileIO<KT, DH>::GSUB > 8192 ? 2 : 4;
  if constexpr (DH == 128) {
    switch (depth) {
      case 1: return launch_score_d<KT, DH, 1>(a, pairs, st);
      case 2: return launch_score_d<KT, DH, 2>(a, pairs, st);
      case 4: return launch_score_d<KT, DH, 4>(a, pairs, st);
      case 8: if constexpr (KT == KEY_FP8) return launch_score_d<KT, DH, 8>(a, pairs, st); break;
      default: break;
    }
  }
  return launch_score_d<KT, DH, DDEF>(a, pairs, st);
}
template <int KT, int DH>
static hipError_t launch_tscore_t(const TopkScoreArgs& a, int pairs, bool contig, hipStream_t st) {
  constexpr int D = TileIO<KT, DH>::GSUB >= 8192 ? 2 : 4;  // about 16 KiB of key loads in flight per wave pair
  if (contig)
    hipLaunchKernelGGL((topk_score_kernel<KT, DH, D, true>), dim3(pairs), dim3(128), 0, st, a);
  else
    hipLaunchKernelGGL((topk_score_kernel<KT, DH, D, false>), dim3(pairs), dim3(128), 0, st, a);
  return hipGetLastError();
}

#define LSA_DISPATCH(FN, KT_, DH_, ...)                                                   \
  do {                                                                                    \
    if (KT_ == KEY_BF16) {                                                                \
      if (DH_ == 128) return FN<KEY_BF16, 128>(__VA_ARGS__);                              \
      if (DH_ == 64) return FN<KEY_BF16, 64>(__VA_ARGS__);                                \
      return FN<KEY_BF16, 32>(__VA_ARGS__);                                               \
    } else if (KT_ == KEY_FP8) {                                                          \
      if (DH_ == 128) return FN<KEY_FP8, 128>(__VA_ARGS__);                               \
      if (DH_ == 64) return FN<KEY_FP8, 64>(__VA_ARGS__);                                 \
      return FN<KEY_FP8, 32>(__VA_ARGS__);                                                \
    } else {                                                                              \
      if (DH_ == 128) return FN<KEY_F32, 128>(__VA_ARGS__);                               \
      if (DH_ == 64) return FN<KEY_F32, 64>(__VA_ARGS__);                                 \
      return FN<KEY_F32, 32>(__VA_ARGS__);                                                \
    }                                                                                     \
  } while (0)

hipError_t launch_score_select(const ScoreArgs& a, int key_kind, int d_h, int pairs, int depth, hipStream_t st) {
  LSA_DISPATCH(launch_score_t, key_kind, d_h, a, pairs, depth, st);
}

hipError_t launch_topk_score(const TopkScoreArgs& a, int key_kind, int d_h, int grid, bool contig, hipStream_t st) {
  LSA_DISPATCH(launch_tscore_t, key_kind, d_h, a, grid, contig, st);
}

}  // namespace lsa
