// Kernel argument blocks and launchers shared between the kernels and the
// C-ABI host layer.
#pragma once

#include "common.hpp"

// Debug builds (-DLSA_DEBUG_CHECKS=1) check every list entry that addresses a row (the
// gather and the top-k scoring of gathered rows) against its sequence's row count, skip
// the access when it is out of range, and count it; lsa_debug_range_errors reports the
// count. Release builds compile none of this.
#ifndef LSA_DEBUG_CHECKS
#define LSA_DEBUG_CHECKS 0
#endif
#define LSA_TOPK_MAX_B 4096
#define TOPK_CONTIG_MAX_B 1024  // sequences of one per-step top-k call over packed subset keys

namespace lsa {

struct ScoreArgs {
  const float* q[LSA_MAX_LAYERS];
  const float* w[LSA_MAX_LAYERS];
  const void* keys[LSA_MAX_LAYERS];
  const float* scale[LSA_MAX_LAYERS];
  uint64_t* mask[LSA_MAX_LAYERS];
  float* score[LSA_MAX_LAYERS];
  const int64_t* key_off;  // [B+1]
  const int64_t* mwo;      // [B+1]
  int64_t word_base;       // mwo[0]
  int64_t words_per_layer; // mwo[B] - mwo[0]
  int64_t total_words;     // L * words_per_layer
  int32_t B, n_h, L;
  float thr;               // logit threshold
  int32_t group;           // pairs per interleave group (grid size is a multiple)
  // one-wave-per-tile kernel: a block's waves take chunks of chunk_words mask words
  int32_t chunk_words;
};

// Histogram of the subset scores per (layer, sequence): bin = top TOPK_HBITS bits
// of the order-preserving key of y. The scoring kernel fills it; the select
// reads the k-th largest score's bin from it.
constexpr int TOPK_HBITS = 11;
constexpr int TOPK_BINS = 1 << TOPK_HBITS;
// Longest sequence (rows) for which the top-k runs without that histogram: every list then fits
// the select's register or reload paths, which count the keys' bins themselves from the scores
// they read anyway, so the scorer keeps no histogram and nothing has to clear one. Calls with a
// longer sequence pass the histogram (hist non-null in both argument blocks).
constexpr int64_t TOPK_NOHIST_MAX_ROWS = 131072;

struct TopkScoreArgs {
  const float* q[LSA_MAX_LAYERS];
  const float* w[LSA_MAX_LAYERS];
  const void* keys[LSA_MAX_LAYERS];     // full key arrays (gathered through idx), or
  const void* sub_keys[LSA_MAX_LAYERS]; // the union rows packed in list order (contiguous mode)
  const float* scale[LSA_MAX_LAYERS];
  float* ys;                // workspace scores [L][rows_total]
  uint32_t* hist;           // workspace [L][B][TOPK_BINS] counts (zeroed before the launch), or null
  const int32_t* idx;       // union lists, region b at key_off[b]
  const int32_t* count;     // [B]
  const int64_t* key_off;   // [B+1]
  int64_t rows_total;
  int32_t B, L, n_h;
};

struct TopkSelectArgs {
  const float* ys;
  const uint32_t* hist;     // the scoring kernel's histograms, or null (the select counts the bins)
  const int32_t* idx;
  const int32_t* count;
  const int64_t* key_off;
  int32_t* out_idx[LSA_MAX_LAYERS];
  float* out_score[LSA_MAX_LAYERS];
  int32_t* out_count;       // [L, B]
  int64_t rows_total;
  int32_t B, k;
};

// Bytes of the top-k workspace: the scores [L][rows], then (256-byte aligned)
// the histograms [L][B][TOPK_BINS].
inline size_t topk_hist_offset(int L, int64_t rows) { return ((size_t)L * (size_t)rows * 4 + 255) & ~(size_t)255; }
inline size_t topk_workspace_bytes(int L, int B, int64_t rows) {
  return topk_hist_offset(L, rows) + (size_t)L * (size_t)B * TOPK_BINS * 4;
}

struct UnionArgs {
  const uint64_t* mask[LSA_MAX_LAYERS];
  const int64_t* key_off;
  const int64_t* mwo;
  int32_t* idx_out;
  int32_t* count_out;
  uint64_t* union_out;
  int32_t L;
  int32_t chunk_words;  // mask words per block: 64, 128, 192 or 256 (set by the launcher)
};

struct GatherArgs {
  const char* pool;
  const int64_t* pool_off;   // [B+1]
  const int32_t* idx;
  const int64_t* idx_off;    // [B]
  const int32_t* count;      // [B]
  char* out;
  const int64_t* out_off;    // [B+1] or null (packed)
  int64_t out_capacity;
  int64_t row_bytes;
  int32_t B;
};

struct ProjArgs {
  const void* h[LSA_MAX_LAYERS];
  const void* w_dq[LSA_MAX_LAYERS];
  const void* w_iuq[LSA_MAX_LAYERS];
  const void* w_w[LSA_MAX_LAYERS];
  float* c[LSA_MAX_LAYERS];
  float* q[LSA_MAX_LAYERS];
  float* w[LSA_MAX_LAYERS];
  int32_t B, d, r, n_h, d_h;
};

// Golden-label mining (nucleus per (token, layer) row, then vote and union).
struct GoldenArgs {
  const float* logits;     // [T][L][row_stride]
  const int32_t* n_valid;  // [T]
  uint64_t* row_mask;      // [T * L][W]
  int32_t* nucleus_size;   // [T * L] or null
  uint64_t* token_golden;  // [T][W] or null
  uint64_t* golden;        // [W]
  char* ws;                // per-segment records, golden_workspace_bytes()
  int64_t row_stride;
  int64_t W;               // ceil(row_stride / 64)
  int32_t T, L;
  float p;
  int32_t theta;           // 1..127
  int32_t S;               // segments per row (set by launch_golden)
};

// Indexer training step (one layer; n_h = 64, d_h = 128 keys in bf16).
constexpr int kTrainDcSlices = 64;  // row slices of W^IUQ in dc = dq W^IUQ (partials [slices][B][r])
struct TrainArgs {
  const void* keys;        // bf16 [rows][128], sequence b at key_off[b]
  const int64_t* key_off;  // [B+1]
  const uint64_t* labels;  // label bits, region b at mwo[b]
  const int64_t* mwo;      // [B+1]
  const void* h;           // bf16 [B][d]
  const void* w_iuq;       // bf16 [n_h*d_h][r]
  const float* c;          // [B][r]
  const float* q;          // [B][n_h][d_h]
  const float* w;          // [B][n_h]
  float* part;             // scan block partials: dq' (the gate factored out) and the loss
  float* dq;               // [B][n_h*d_h]
  float* dw;               // [B][n_h]
  float* dc;               // [B][r]
  float* dcp;              // dc partials [kTrainDcSlices][B][r], 16-byte aligned
  float* loss;             // [1]
  float* g_dq;             // [r][d]
  float* g_iuq;            // [n_h*d_h][r]
  float* g_w;              // [n_h][d]
  int64_t nblk;            // scan blocks
  int32_t tpb;             // 32-entry tiles per scan block
  int32_t B, d, r;
  float gamma, alpha, inv_total;
};

hipError_t launch_score_select(const ScoreArgs& a, int key_kind, int d_h, int pairs, int depth, hipStream_t st);
// one wave per tile, keys loaded straight into LDS (bf16 and fp8 keys)
bool score_stream_supported(int key_kind, int d_h);
// guard: the hi-only pass with a per-tile refine (no sigmoid scores)
hipError_t launch_score_stream(const ScoreArgs& a, int key_kind, int d_h, int waves, int ring, bool guard,
                               hipStream_t st);
// contig: the keys come from sub_keys (packed union rows), else gathered through idx
hipError_t launch_topk_score(const TopkScoreArgs& a, int key_kind, int d_h, int grid, bool contig, hipStream_t st);
hipError_t launch_topk_hist_zero(uint32_t* hist, int64_t n, hipStream_t st);
hipError_t launch_topk_select(const TopkSelectArgs& a, int L, hipStream_t st);
hipError_t launch_union_compact(const UnionArgs& a, int B, int64_t max_words, int cus, hipStream_t st);
hipError_t launch_gather(const GatherArgs& a, int grid, int rows_per_wave, hipStream_t st);
// Debug builds: the out-of-range list entries each file's kernels have skipped since the last
// call (the count is read, then cleared; synchronous).
hipError_t gather_take_range_errors(unsigned int* out);
hipError_t topk_take_range_errors(unsigned int* out);

hipError_t launch_project(const ProjArgs& a, int L, bool f32, hipStream_t st);
hipError_t launch_project_packed(const ProjArgs& a, int L, hipStream_t st);
// One bf16 layer with each reduction split over two blocks that add into zeroed outputs (a grid of
// twice the blocks, for a single layer on a large device).
hipError_t launch_project_split2(const ProjArgs& a, hipStream_t st);
size_t golden_workspace_bytes(int64_t rows, int64_t row_stride);
int64_t train_scan_blocks(const int64_t* key_off_host, int B, int* tiles_per_block);
size_t train_workspace_bytes(int B, int r, int64_t nblk);
struct TrainWs {
  float *c, *q, *w, *dq, *dw, *dc, *dcp, *part;
  size_t bytes;
};
TrainWs train_carve(void* ws, int B, int r, int64_t nblk);
hipError_t launch_train_zero(float* p, int64_t n, hipStream_t st);
hipError_t launch_train(const TrainArgs& a, hipStream_t st);
hipError_t launch_golden(const GoldenArgs& a, hipStream_t st);
hipError_t launch_pack_weights(const void* w, int rows, int K, void* out, hipStream_t st);

// ------------------------------------------------------------ block helpers
// Exclusive prefix sum over the threads of a block (blockDim.x a multiple of
// 64, at most 1024). Every thread of the block must call it.
__device__ __forceinline__ int64_t block_exclusive_scan(int64_t v, int64_t* total) {
  __shared__ int64_t wsum[16];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nwv = blockDim.x >> 6;
  int64_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int64_t off = 0, tot = 0;
  for (int i = 0; i < nwv; ++i) {
    const int64_t s = wsum[i];
    off += i < w ? s : 0;
    tot += s;
  }
  __syncthreads();
  if (total) *total = tot;
  return off + x - v;
}

// tp[b] = tiles of the lists before b, rp[b] = entries of the lists before b
// (b = 0..B; the caller keeps the totals below 2^31).
__device__ __forceinline__ void block_list_prefix(const int32_t* __restrict__ count, int B, int32_t* tp, int32_t* rp) {
  const int nt = blockDim.x, tid = threadIdx.x;
  const int per = (B + nt - 1) / nt;
  const int lo = min(B, tid * per), hi = min(B, lo + per);
  int64_t s = 0;
  for (int b = lo; b < hi; ++b) s += ((int64_t)(count[b] + 31) >> 5) << 32 | (uint32_t)count[b];
  int64_t tot;
  int64_t run = block_exclusive_scan(s, &tot);  // tiles in the high word, entries in the low word
  for (int b = lo; b < hi; ++b) {
    tp[b] = (int32_t)(run >> 32);
    rp[b] = (int32_t)(uint32_t)run;
    run += ((int64_t)(count[b] + 31) >> 5) << 32 | (uint32_t)count[b];
  }
  if (tid == 0) {
    tp[B] = (int32_t)(tot >> 32);
    rp[B] = (int32_t)(uint32_t)tot;
  }
  __syncthreads();
}

// tp[b] = sum over b' < b of ceil(count[b'] / 32), for b = 0..B (B <= LSA_TOPK_MAX_B).
__device__ __forceinline__ void block_tile_prefix(const int32_t* __restrict__ count, int B, int32_t* tp) {
  const int nt = blockDim.x, tid = threadIdx.x;
  const int per = (B + nt - 1) / nt;
  const int lo = min(B, tid * per), hi = min(B, lo + per);
  int64_t s = 0;
  for (int b = lo; b < hi; ++b) s += (count[b] + 31) >> 5;
  int64_t tot;
  int64_t run = block_exclusive_scan(s, &tot);
  for (int b = lo; b < hi; ++b) {
    tp[b] = (int32_t)run;
    run += (count[b] + 31) >> 5;
  }
  if (tid == 0) tp[B] = (int32_t)tot;
  __syncthreads();
}

}  // namespace lsa
