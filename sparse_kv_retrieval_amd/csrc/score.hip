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
#include "kernels.hpp"
#include "scorer.hpp"

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

// Sequence table lookups. For up to SEQ_TAB entries the key and word offsets
// are copied to LDS once per block. A lookup is then an LDS read, which never
// waits on the vector-memory counter that tracks the key DMAs.
constexpr int SEQ_TAB = 256;

struct SeqTab {
  const int64_t* koff;  // LDS or global
  const int64_t* mwo;
};

// Wave-uniform cursor over the mask words of one wave: (layer, sequence, word).
// It advances one word at a time, so there is no division or search in the
// steady state. A search runs only when the cursor is placed.
struct WordCursor {
  int l, b;
  int64_t word;     // word index in the mask layout
  int64_t seq_hi;   // first word after sequence b
  int64_t e0;       // entry index (within sequence b) of the word's first bit
  int64_t row0, nb; // sequence b's first key row and entry count

  __device__ __forceinline__ void load_seq(const SeqTab& t) {
    const int64_t lo = uni(t.mwo[b]);
    seq_hi = uni(t.mwo[b + 1]);
    row0 = uni(t.koff[b]);
    nb = uni(t.koff[b + 1]) - row0;
    e0 = (word - lo) * 64;
  }
  __device__ __forceinline__ void place(const ScoreArgs& a, const SeqTab& t, int64_t gw) {
    l = uni((int32_t)(gw / a.words_per_layer));
    word = uni(a.word_base + (gw - (int64_t)l * a.words_per_layer));
    b = uni(upper_seq(t.mwo, a.B, word));
    load_seq(t);
  }
  __device__ __forceinline__ void next(const ScoreArgs& a, const SeqTab& t) {
    ++word;
    e0 += 64;
    if (word == seq_hi) {
      if (word == a.word_base + a.words_per_layer) {
        ++l;
        word = a.word_base;
        b = 0;
      } else {
        ++b;
      }
      while (uni(t.mwo[b + 1]) == uni(t.mwo[b])) ++b;  // skip empty sequences
      load_seq(t);
    }
  }
};

// Score + select: keys streamed HBM -> registers -> LDS -> MFMA, two waves per tile.
//
// A block is one pair of waves and owns a contiguous run of mask words. Each
// word is two 32-entry tiles. Wave h loads half of every tile with coalesced
// 16-byte vector loads (each load instruction covers 1 KiB of contiguous key
// rows) and keeps D tiles in flight in registers. When a tile's turn comes, it
// writes the tile into one of two LDS stages. fp8 keys are widened to bf16 on
// the way (exact), so both waves then run the bf16 MFMA on the same
// operands. In LDS, 16-byte chunk c of row r sits at position c ^ (r % CPR), so
// the operand reads (lane n reads row n) are free of bank conflicts.
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
};

template <int KT, int DH, int D>
__global__ __launch_bounds__(128) void score_select_kernel(const ScoreArgs a) {
  using IO = TileIO<KT, DH>;
  using S_t = Scorer<KT == KEY_F32 ? KEY_F32 : KEY_BF16, DH, 1>;
  static_assert(S_t::ROW_BYTES == IO::LRB, "LDS row layout");
  __shared__ __attribute__((aligned(16))) char stage[2][IO::LSUB];
  __shared__ float xpart[2][32];
  __shared__ int64_t tab[2][SEQ_TAB + 1];

  const int lane = threadIdx.x & 63, g = lane >> 5, n = lane & 31;
  const int h = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // which half of the heads
  SeqTab t{a.key_off, a.mwo};
  if (a.B < SEQ_TAB) {
    for (int i = threadIdx.x; i <= a.B; i += 128) {
      tab[0][i] = a.key_off[i];
      tab[1][i] = a.mwo[i];
    }
    __syncthreads();
    t.koff = tab[0];
    t.mwo = tab[1];
  }
  const int64_t np = gridDim.x;
  const int64_t gbeg = (int64_t)blockIdx.x * a.total_words / np;
  const int64_t gend = ((int64_t)blockIdx.x + 1) * a.total_words / np;
  const int J = (int)(2 * (gend - gbeg));  // tiles of this pair
  if (J == 0) return;

  // This wave's load instructions: [i0, i0 + NLW), or none for 1 KiB tiles on wave 1.
  const int i0 = IO::NLI >= 2 ? h * IO::NLW : 0;
  const bool loads = IO::NLI >= 2 || h == 0;
  // per instruction: row within the tile, and the stored chunk of that row
  int lrow[IO::NLW], lchunk[IO::NLW];
#pragma unroll
  for (int i = 0; i < IO::NLW; ++i) {
    const int p = (i0 + i) * 1024 + lane * 16;
    lrow[i] = p / IO::GRB;
    lchunk[i] = (p % IO::GRB) / 16;
  }

  u32x4 R[D][IO::NLW];
  float SC[D];
  WordCursor ic, cc;
  ic.place(a, t, gbeg);
  cc = ic;

  S_t S;
  int cur_l = -1, cur_b = -1;
  float pprev = 0.0f;
  bool vprev = false;
  int64_t rprev = 0, wprev = 0;
  int lprev = 0;
  uint32_t bits0 = 0;

#define LSA_LOAD_TILE(SLOT, JJ)                                                                     \
  do {                                                                                              \
    const int64_t e_ = ic.e0 + ((JJ) & 1) * 32;                                                     \
    const int64_t last_ = ic.row0 + ic.nb - 1;                                                      \
    const char* kb_ = (const char*)a.keys[ic.l];                                                    \
    if (loads) {                                                                                    \
      _Pragma("unroll") for (int i = 0; i < IO::NLW; ++i) {                                         \
        const int64_t row_ = min(ic.row0 + e_ + lrow[i], last_);                                    \
        R[SLOT][i] = __builtin_nontemporal_load((const u32x4*)(kb_ + row_ * IO::GRB + lchunk[i] * 16)); \
      }                                                                                             \
    }                                                                                               \
    if constexpr (KT == KEY_FP8) SC[SLOT] = a.scale[ic.l][min(ic.row0 + e_ + n, last_)];            \
    if ((JJ) & 1) ic.next(a, t);                                                                    \
  } while (0)

#pragma unroll
  for (int s = 0; s < D; ++s)
    if (s < J) LSA_LOAD_TILE(s, s);

  for (int j0 = 0; j0 < J; j0 += D) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      const int j = j0 + s;
      if (j >= J) break;
      char* st = &stage[j & 1][0];
      // write this wave's half of tile j into LDS (waits for its loads)
      if (loads) {
#pragma unroll
        for (int i = 0; i < IO::NLW; ++i) {
          const int r = lrow[i];
          char* rowp = st + r * IO::LRB;
          if constexpr (KT == KEY_FP8) {
            const u32x4 v = R[s][i];
            const u32x2 b0 = e4m3x4_to_bf16x4(v[0]), b1 = e4m3x4_to_bf16x4(v[1]);
            const u32x2 b2 = e4m3x4_to_bf16x4(v[2]), b3 = e4m3x4_to_bf16x4(v[3]);
            const int c0 = 2 * lchunk[i], c1 = c0 + 1;
            *(u32x4*)(rowp + ((c0 ^ (r % IO::LCPR)) * 16)) = u32x4{b0[0], b0[1], b1[0], b1[1]};
            *(u32x4*)(rowp + ((c1 ^ (r % IO::LCPR)) * 16)) = u32x4{b2[0], b2[1], b3[0], b3[1]};
          } else {
            *(u32x4*)(rowp + ((lchunk[i] ^ (r % IO::LCPR)) * 16)) = R[s][i];
          }
        }
      }
      float scale = 1.0f;
      if constexpr (KT == KEY_FP8) scale = SC[s];
      // refill this slot with tile j + D
      if (j + D < J) LSA_LOAD_TILE(s, j + D);
      lds_barrier();  // tile j complete in LDS; wave 1's partial of tile j-1 visible
      S.read_keys_lds(st);

      if (h == 0 && j > 0) {
        // finish tile j-1: both halves of the head sum, threshold, ballot, stores
        const float x = pprev + xpart[(j - 1) & 1][n];
        const uint32_t bits = (uint32_t)__ballot(vprev && x >= a.thr);
        float* so = a.score[lprev];
        if (so != nullptr && g == 0 && vprev) so[rprev] = 1.0f / (1.0f + __expf(-x));
        if ((j - 1) & 1) {
          if (lane == 0) a.mask[lprev][wprev] = (uint64_t)bits0 | ((uint64_t)bits << 32);
        } else {
          bits0 = bits;
        }
      }
      if (cc.l != cur_l || cc.b != cur_b) {
        S.load_query(a.q[cc.l], a.w[cc.l], cc.b, a.n_h, 32 * h);
        cur_l = cc.l;
        cur_b = cc.b;
      }
      f32x16 acc[1];
      S.mma(acc);
      float p = S.partial(acc);
      p += __shfl_xor(p, 32);
      if constexpr (KT == KEY_FP8) p *= scale;
      const int64_t se = cc.e0 + (j & 1) * 32 + n;
      if (h == 1) {
        if (g == 0) xpart[j & 1][n] = p;
      } else {
        pprev = p;
        vprev = se < cc.nb;
        rprev = cc.row0 + se;
        wprev = cc.word;
        lprev = cc.l;
      }
      if (j & 1) cc.next(a, t);
    }
  }
#undef LSA_LOAD_TILE
  lds_barrier();
  if (h == 0) {
    const int j = J;
    const float x = pprev + xpart[(j - 1) & 1][n];
    const uint32_t bits = (uint32_t)__ballot(vprev && x >= a.thr);
    float* so = a.score[lprev];
    if (so != nullptr && g == 0 && vprev) so[rprev] = 1.0f / (1.0f + __expf(-x));
    if (lane == 0) a.mask[lprev][wprev] = (uint64_t)bits0 | ((uint64_t)bits << 32);  // J is even: tile J-1 is odd
  }
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
  __device__ __forceinline__ void load_seq(const TopkScoreArgs& a, const int32_t* tp) {
    nt = uni(tp[b + 1]) - uni(tp[b]);
    base = uni(a.key_off[b]);
    cnt = uni(a.count[b]);
  }
  __device__ __forceinline__ void place(const TopkScoreArgs& a, const int32_t* tp, int64_t t) {
    const int64_t tpl = uni(tp[a.B]);
    l = uni((int32_t)(t / tpl));
    const int32_t tt = (int32_t)(t - (int64_t)l * tpl);
    b = uni(upper_seq(tp, a.B, tt));
    jt = tt - uni(tp[b]);
    load_seq(a, tp);
  }
  __device__ __forceinline__ void next(const TopkScoreArgs& a, const int32_t* tp) {
    if (++jt < nt) return;
    jt = 0;
    do {
      if (++b == a.B) {
        b = 0;
        ++l;
      }
    } while (uni(tp[b + 1]) == uni(tp[b]));
    load_seq(a, tp);
  }
};

template <int KT, int DH, int D>
__global__ __launch_bounds__(128) void topk_score_kernel(const TopkScoreArgs a) {
  using IO = TileIO<KT, DH>;
  using S_t = Scorer<KT == KEY_F32 ? KEY_F32 : KEY_BF16, DH, 1>;
  static_assert(IO::GRB == 16 * (IO::GRB / 16), "row size");
  __shared__ __attribute__((aligned(16))) char stage[2][IO::LSUB];
  __shared__ float xpart[2][32];
  __shared__ int32_t tp[LSA_TOPK_MAX_B + 1];

  const int lane = threadIdx.x & 63, g = lane >> 5, n = lane & 31;
  const int h = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  block_tile_prefix(a.count, a.B, tp);
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
  xc.place(a, tp, t0);
  ic = xc;
  cc = xc;

#define LSA_LOAD_IDX(SLOT)                                                                     \
  do {                                                                                         \
    const int32_t e_ = xc.jt * 32;                                                             \
    const int32_t* il_ = a.idx + xc.base;                                                      \
    _Pragma("unroll") for (int i = 0; i < IO::NLW; ++i) IX[SLOT][i] = il_[min(e_ + lrow[i], xc.cnt - 1)]; \
    if constexpr (KT == KEY_FP8) IXS[SLOT] = il_[min(e_ + n, xc.cnt - 1)];                     \
    xc.next(a, tp);                                                                            \
  } while (0)
#define LSA_LOAD_KEYS(SLOT, XSLOT)                                                             \
  do {                                                                                         \
    const char* kb_ = (const char*)a.keys[ic.l] + ic.base * IO::GRB;                           \
    if (loads) {                                                                               \
      _Pragma("unroll") for (int i = 0; i < IO::NLW; ++i)                                      \
        R[SLOT][i] = __builtin_nontemporal_load(                                               \
            (const u32x4*)(kb_ + (int64_t)IX[XSLOT][i] * IO::GRB + lchunk[i] * 16));           \
    }                                                                                          \
    if constexpr (KT == KEY_FP8) SC[SLOT] = a.scale[ic.l][ic.base + IXS[XSLOT]];               \
    ic.next(a, tp);                                                                            \
  } while (0)

  // prologue: indices for tiles 0 .. 2D-1, keys for tiles 0 .. D-1
#pragma unroll
  for (int s = 0; s < 2 * D; ++s)
    if (s < J) LSA_LOAD_IDX(s);
#pragma unroll
  for (int s = 0; s < D; ++s)
    if (s < J) LSA_LOAD_KEYS(s, s);

  S_t S;
  int cur_l = -1, cur_b = -1;
  float pprev = 0.0f;
  bool vprev = false;
  int64_t oprev = 0;

  for (int j0 = 0; j0 < J; j0 += 2 * D) {
#pragma unroll
    for (int s = 0; s < 2 * D; ++s) {
      const int j = j0 + s;
      if (j >= J) break;
      const int rs = s % D;  // register slot of tile j
      char* st = &stage[j & 1][0];
      if (loads) {
#pragma unroll
        for (int i = 0; i < IO::NLW; ++i) {
          const int r = lrow[i];
          char* rowp = st + r * IO::LRB;
          if constexpr (KT == KEY_FP8) {
            const u32x4 v = R[rs][i];
            const u32x2 b0 = e4m3x4_to_bf16x4(v[0]), b1 = e4m3x4_to_bf16x4(v[1]);
            const u32x2 b2 = e4m3x4_to_bf16x4(v[2]), b3 = e4m3x4_to_bf16x4(v[3]);
            const int c0 = 2 * lchunk[i], c1 = c0 + 1;
            *(u32x4*)(rowp + ((c0 ^ (r % IO::LCPR)) * 16)) = u32x4{b0[0], b0[1], b1[0], b1[1]};
            *(u32x4*)(rowp + ((c1 ^ (r % IO::LCPR)) * 16)) = u32x4{b2[0], b2[1], b3[0], b3[1]};
          } else {
            *(u32x4*)(rowp + ((lchunk[i] ^ (r % IO::LCPR)) * 16)) = R[rs][i];
          }
        }
      }
      float scale = 1.0f;
      if constexpr (KT == KEY_FP8) scale = SC[rs];
      if (j + D < J) LSA_LOAD_KEYS(rs, (s + D) % (2 * D));
      if (j + 2 * D < J) LSA_LOAD_IDX(s);
      lds_barrier();
      S.read_keys_lds(st);
      if (h == 0 && j > 0) {
        const float y = pprev + xpart[(j - 1) & 1][n];
        if (g == 0 && vprev) a.ys[oprev] = y;
      }
      if (cc.l != cur_l || cc.b != cur_b) {
        S.load_query(a.q[cc.l], a.w[cc.l], cc.b, a.n_h, 32 * h);
        cur_l = cc.l;
        cur_b = cc.b;
      }
      f32x16 acc[1];
      S.mma(acc);
      float p = S.partial(acc);
      p += __shfl_xor(p, 32);
      if constexpr (KT == KEY_FP8) p *= scale;
      const int32_t e = cc.jt * 32 + n;
      if (h == 1) {
        if (g == 0) xpart[j & 1][n] = p;
      } else {
        pprev = p;
        vprev = e < cc.cnt;
        oprev = (int64_t)cc.l * a.rows_total + cc.base + e;
      }
      cc.next(a, tp);
    }
  }
#undef LSA_LOAD_IDX
#undef LSA_LOAD_KEYS
  lds_barrier();
  if (h == 0) {
    const float y = pprev + xpart[(J - 1) & 1][n];
    if (g == 0 && vprev) a.ys[oprev] = y;
  }
}

// ------------------------------------------------------------------ launch
template <int KT, int DH, int NHB>
static hipError_t launch_score_t(const ScoreArgs& a, int pairs, hipStream_t st) {
  // one block = one pair of waves; D tiles in flight per wave in registers
  constexpr int D = TileIO<KT, DH>::GSUB > 8192 ? 2 : 4;
  hipLaunchKernelGGL((score_select_kernel<KT, DH, D>), dim3(pairs), dim3(128), 0, st, a);
  return hipGetLastError();
}
template <int KT, int DH, int NHB>
static hipError_t launch_tscore_t(const TopkScoreArgs& a, int pairs, hipStream_t st) {
  constexpr int D = TileIO<KT, DH>::GSUB >= 8192 ? 2 : 4;
  hipLaunchKernelGGL((topk_score_kernel<KT, DH, D>), dim3(pairs), dim3(128), 0, st, a);
  return hipGetLastError();
}

#define LSA_DISPATCH(FN, KT_, DH_, NHB_, ...)                                       \
  do {                                                                              \
    if (KT_ == KEY_BF16) {                                                          \
      if (DH_ == 128) return NHB_ == 1 ? FN<KEY_BF16, 128, 1>(__VA_ARGS__) : FN<KEY_BF16, 128, 2>(__VA_ARGS__); \
      if (DH_ == 64) return NHB_ == 1 ? FN<KEY_BF16, 64, 1>(__VA_ARGS__) : FN<KEY_BF16, 64, 2>(__VA_ARGS__);    \
      return NHB_ == 1 ? FN<KEY_BF16, 32, 1>(__VA_ARGS__) : FN<KEY_BF16, 32, 2>(__VA_ARGS__);                   \
    } else if (KT_ == KEY_FP8) {                                                    \
      if (DH_ == 128) return NHB_ == 1 ? FN<KEY_FP8, 128, 1>(__VA_ARGS__) : FN<KEY_FP8, 128, 2>(__VA_ARGS__);   \
      if (DH_ == 64) return NHB_ == 1 ? FN<KEY_FP8, 64, 1>(__VA_ARGS__) : FN<KEY_FP8, 64, 2>(__VA_ARGS__);      \
      return NHB_ == 1 ? FN<KEY_FP8, 32, 1>(__VA_ARGS__) : FN<KEY_FP8, 32, 2>(__VA_ARGS__);                     \
    } else {                                                                        \
      if (DH_ == 128) return NHB_ == 1 ? FN<KEY_F32, 128, 1>(__VA_ARGS__) : FN<KEY_F32, 128, 2>(__VA_ARGS__);   \
      if (DH_ == 64) return NHB_ == 1 ? FN<KEY_F32, 64, 1>(__VA_ARGS__) : FN<KEY_F32, 64, 2>(__VA_ARGS__);      \
      return NHB_ == 1 ? FN<KEY_F32, 32, 1>(__VA_ARGS__) : FN<KEY_F32, 32, 2>(__VA_ARGS__);                     \
    }                                                                               \
  } while (0)

hipError_t launch_score_select(const ScoreArgs& a, int key_kind, int d_h, int pairs, hipStream_t st) {
  const int nhb = a.n_h > 32 ? 2 : 1;
  LSA_DISPATCH(launch_score_t, key_kind, d_h, nhb, a, pairs, st);
}

hipError_t launch_topk_score(const TopkScoreArgs& a, int key_kind, int d_h, int grid, hipStream_t st) {
  const int nhb = a.n_h > 32 ? 2 : 1;
  LSA_DISPATCH(launch_tscore_t, key_kind, d_h, nhb, a, grid, st);
}

}  // namespace lsa
