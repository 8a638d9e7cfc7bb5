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

template <int KT, int DH, int NHB>
__global__ __launch_bounds__(256) void score_select_kernel(const ScoreArgs a) {
  using S_t = Scorer<KT, DH, NHB>;
  const int lane = threadIdx.x & 63, g = lane >> 5, n = lane & 31;
  const int wave_in_block = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nw = (int64_t)gridDim.x * (blockDim.x >> 6);
  const int64_t wid = (int64_t)blockIdx.x * (blockDim.x >> 6) + wave_in_block;
  int64_t gw = wid * a.total_words / nw;
  const int64_t gend = (wid + 1) * a.total_words / nw;

  S_t S;
  int cur_l = -1, cur_b = -1;
  int64_t seq_lo = 0, seq_hi = -1, row0 = 0, nb = 0;
  const char* keys = nullptr;
  for (; gw < gend; ++gw) {
    const int l = (int)(gw / a.words_per_layer);
    const int64_t word = a.word_base + (gw - (int64_t)l * a.words_per_layer);
    if (l != cur_l || word < seq_lo || word >= seq_hi) {
      const int b = upper_seq(a.mwo, a.B, word);
      seq_lo = a.mwo[b];
      seq_hi = a.mwo[b + 1];
      row0 = a.key_off[b];
      nb = a.key_off[b + 1] - row0;
      keys = (const char*)a.keys[l];
      if (l != cur_l || b != cur_b) {
        S.load_query(a.q[l], a.w[l], b, a.n_h);
        cur_l = l;
        cur_b = b;
      }
    }
    const int64_t s0 = (word - seq_lo) * 64;
    uint32_t bits[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int64_t s = s0 + sub * 32 + n;
      const bool valid = s < nb;
      const int64_t row = row0 + (valid ? s : 0);
      S.load_keys(keys + row * S_t::ROW_BYTES + g * S_t::HALF_BYTES, valid);
      f32x16 acc[NHB];
      S.mma(acc);
      float x = S.logit(acc);
      if constexpr (KT == KEY_FP8) x *= valid ? a.scale[l][row] : 0.0f;
      bits[sub] = (uint32_t)__ballot(valid && x >= a.thr);
      float* so = a.score[l];
      if (so != nullptr && g == 0 && valid) so[row] = 1.0f / (1.0f + __expf(-x));
    }
    if (lane == 0) a.mask[l][word] = (uint64_t)bits[0] | ((uint64_t)bits[1] << 32);
  }
}

// Gathered scoring for the top-k: y = sum_j w'_j ReLU(q'_j . K_s) for each s in
// the union list ([BLOG] §3.2: the native indexer works only inside the loaded
// subset). The 32-entry tiles of all (layer, sequence) lists are numbered
// consecutively, and each wave takes a contiguous run of tiles.
template <int KT, int DH, int NHB>
__global__ __launch_bounds__(256) void topk_score_kernel(const TopkScoreArgs a) {
  using S_t = Scorer<KT, DH, NHB>;
  __shared__ int32_t tp[LSA_TOPK_MAX_B + 1];  // tile prefix over sequences
  const int lane = threadIdx.x & 63, g = lane >> 5, n = lane & 31;
  block_tile_prefix(a.count, a.B, tp);
  const int64_t tiles_per_layer = tp[a.B];
  const int64_t total = tiles_per_layer * a.L;
  const int wave_in_block = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nw = (int64_t)gridDim.x * (blockDim.x >> 6);
  const int64_t wid = (int64_t)blockIdx.x * (blockDim.x >> 6) + wave_in_block;
  int64_t t = wid * total / nw;
  const int64_t tend = (wid + 1) * total / nw;

  S_t S;
  int cur_l = -1, cur_b = -1;
  for (; t < tend; ++t) {
    const int l = (int)(t / tiles_per_layer);
    const int32_t tt = (int32_t)(t - (int64_t)l * tiles_per_layer);
    const int b = upper_seq(tp, a.B, tt);
    if (l != cur_l || b != cur_b) {
      S.load_query(a.q[l], a.w[l], b, a.n_h);
      cur_l = l;
      cur_b = b;
    }
    const int64_t base = a.key_off[b];
    const int32_t cnt = a.count[b];
    const int32_t i = (tt - tp[b]) * 32 + n;
    const bool valid = i < cnt;
    const int64_t row = base + (valid ? a.idx[base + i] : 0);
    S.load_keys((const char*)a.keys[l] + row * S_t::ROW_BYTES + g * S_t::HALF_BYTES, valid);
    f32x16 acc[NHB];
    S.mma(acc);
    float y = S.logit(acc);
    if constexpr (KT == KEY_FP8) y *= valid ? a.scale[l][row] : 0.0f;
    if (g == 0 && valid) a.ys[(int64_t)l * a.rows_total + base + i] = y;
  }
}

// ------------------------------------------------------------------ launch
template <int KT, int DH, int NHB>
static hipError_t launch_score_t(const ScoreArgs& a, int grid, hipStream_t st) {
  hipLaunchKernelGGL((score_select_kernel<KT, DH, NHB>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}
template <int KT, int DH, int NHB>
static hipError_t launch_tscore_t(const TopkScoreArgs& a, int grid, hipStream_t st) {
  hipLaunchKernelGGL((topk_score_kernel<KT, DH, NHB>), dim3(grid), dim3(256), 0, st, a);
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

hipError_t launch_score_select(const ScoreArgs& a, int key_kind, int d_h, int grid, hipStream_t st) {
  const int nhb = a.n_h > 32 ? 2 : 1;
  LSA_DISPATCH(launch_score_t, key_kind, d_h, nhb, a, grid, st);
}

hipError_t launch_topk_score(const TopkScoreArgs& a, int key_kind, int d_h, int grid, hipStream_t st) {
  const int nhb = a.n_h > 32 ? 2 : 1;
  LSA_DISPATCH(launch_tscore_t, key_kind, d_h, nhb, a, grid, st);
}

}  // namespace lsa
