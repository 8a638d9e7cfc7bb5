// Top-k inside the loaded subset: the second level of the two-level selection
// ([BLOG] §3.2 of the FlashMemory-DeepSeek-V4 write-up: the native Lightning
// Indexer picks the final top-k core entries inside C^MemComp).
//
// One block per (sequence, layer). The scores y are in the workspace, in
// subset order, which is ascending entry order. The k-th largest key is found
// by a 4-pass MSB-first radix select over order-preserving uint32 keys, using
// 256-bin LDS histograms. A final ordered pass keeps every entry above the
// k-th key, plus the lowest-index entries equal to it. That matches the
// (-y, s) order, and the output stays ascending because the pass walks the
// list in order.
#include "kernels.hpp"

namespace lsa {

static constexpr int TS_THREADS = 1024;

__global__ __launch_bounds__(TS_THREADS) void topk_select_kernel(const TopkSelectArgs a) {
  const int b = blockIdx.x, l = blockIdx.y, tid = threadIdx.x;
  const int64_t base = a.key_off[b];
  const int32_t M = a.count[b];
  const int32_t k = a.k;
  const float* ys = a.ys + (int64_t)l * a.rows_total + base;
  const int32_t* idx = a.idx + base;
  int32_t* out = a.out_idx[l] + (int64_t)b * k;
  float* outs = a.out_score[l] ? a.out_score[l] + (int64_t)b * k : nullptr;

  if (M <= k) {
    for (int32_t i = tid; i < k; i += TS_THREADS) {
      out[i] = i < M ? idx[i] : -1;
      if (outs) outs[i] = i < M ? ys[i] : -INFINITY;
    }
    if (tid == 0) a.out_count[l * gridDim.x + b] = M;
    return;
  }

  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh_digit, sh_krem;
  uint32_t prefix = 0, pmask = 0;
  uint32_t krem = (uint32_t)k;  // how many of the remaining candidates to take
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int32_t i = tid; i < M; i += TS_THREADS) {
      const uint32_t u = order_key(ys[i]);
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // lane j owns bins 4j..4j+3; suffix sums from the top bin down
      uint32_t s4[4], own = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) { s4[i] = hist[4 * tid + i]; own += s4[i]; }
      uint32_t suf = own;  // inclusive suffix over lanes >= tid
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_down(suf, o);
        if (tid + o < 64) suf += y;
      }
      const uint32_t above = suf - own;  // candidates in bins of higher lanes
      if (above < krem && krem <= suf) {
        uint32_t cum = above;
        for (int i = 3; i >= 0; --i) {
          if (cum + s4[i] >= krem) {
            sh_digit = 4 * tid + i;
            sh_krem = krem - cum;
            break;
          }
          cum += s4[i];
        }
      }
    }
    __syncthreads();
    prefix |= sh_digit << shift;
    pmask |= 255u << shift;
    krem = sh_krem;
    __syncthreads();
  }
  const uint32_t T = prefix;  // key of the k-th largest score; take `krem` entries equal to it

  int64_t run_out = 0, run_eq = 0;
  for (int32_t base_i = 0; base_i < M; base_i += TS_THREADS) {
    const int32_t i = base_i + tid;
    const bool in = i < M;
    const float y = in ? ys[i] : 0.0f;
    const uint32_t u = in ? order_key(y) : 0u;
    const bool gt = in && u > T;
    const bool eq = in && u == T;
    int64_t tot_eq, tot_take;
    const int64_t eq_before = run_eq + block_exclusive_scan(eq ? 1 : 0, &tot_eq);
    const bool take = gt || (eq && eq_before < (int64_t)krem);
    const int64_t pos = run_out + block_exclusive_scan(take ? 1 : 0, &tot_take);
    if (take) {
      out[pos] = idx[i];
      if (outs) outs[pos] = y;
    }
    run_out += tot_take;
    run_eq += tot_eq;
  }
  if (tid == 0) a.out_count[l * gridDim.x + b] = k;
}

hipError_t launch_topk_select(const TopkSelectArgs& a, int L, hipStream_t st) {
  hipLaunchKernelGGL(topk_select_kernel, dim3(a.B, L), dim3(TS_THREADS), 0, st, a);
  return hipGetLastError();
}

}  // namespace lsa
