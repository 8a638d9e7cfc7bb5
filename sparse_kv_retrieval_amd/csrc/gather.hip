// Load step: copy the selected compressed-KV rows into a compact buffer (the
// hyper.ai digest of FlashMemory-DeepSeek-V4, "方法": C^MemComp is loaded into
// GPU memory). This version copies HBM to HBM.
//
// Each block computes, in LDS, where every sequence's rows land: a prefix sum
// of min(count, capacity) in explicit mode, or of count in packed mode. The
// output rows are then numbered 0..total-1 and the waves stride over them.
// One wave copies one row with 16-byte non-temporal loads and stores, so a
// 1 KiB latent row is a single fully coalesced wave access.
#include "kernels.hpp"

namespace lsa {

static constexpr int GA_THREADS = 256;

__global__ __launch_bounds__(GA_THREADS) void gather_kernel(const GatherArgs a) {
  __shared__ int64_t pre[LSA_TOPK_MAX_B + 1];
  const int tid = threadIdx.x;
  {
    const int per = (a.B + GA_THREADS - 1) / GA_THREADS;
    const int lo = min(a.B, tid * per), hi = min(a.B, lo + per);
    auto rows_of = [&](int b) -> int64_t {
      int64_t c = a.count[b];
      if (a.out_off) {
        const int64_t cap = a.out_off[b + 1] - a.out_off[b];
        c = c < cap ? c : cap;
      }
      return c;
    };
    int64_t s = 0;
    for (int b = lo; b < hi; ++b) s += rows_of(b);
    int64_t tot;
    int64_t run = block_exclusive_scan(s, &tot);
    for (int b = lo; b < hi; ++b) {
      pre[b] = run;
      run += rows_of(b);
    }
    if (tid == 0) pre[a.B] = tot;
    __syncthreads();
  }
  const int64_t total = pre[a.B];
  const int lane = tid & 63;
  const int wave_in_block = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t nw = (int64_t)gridDim.x * (GA_THREADS / 64);
  for (int64_t r = (int64_t)blockIdx.x * (GA_THREADS / 64) + wave_in_block; r < total; r += nw) {
    const int b = upper_seq(pre, a.B, r);
    const int64_t i = r - pre[b];
    const int64_t dst_row = a.out_off ? a.out_off[b] + i : r;
    if (dst_row >= a.out_capacity) continue;
    const int64_t src_row = a.pool_off[b] + a.idx[a.idx_off[b] + i];
    const u32x4* src = (const u32x4*)(a.pool + src_row * a.row_bytes);
    u32x4* dst = (u32x4*)(a.out + dst_row * a.row_bytes);
    const int64_t n16 = a.row_bytes >> 4;
    for (int64_t j = lane; j < n16; j += 64) __builtin_nontemporal_store(__builtin_nontemporal_load(src + j), dst + j);
  }
}

hipError_t launch_gather(const GatherArgs& a, int grid, hipStream_t st) {
  hipLaunchKernelGGL(gather_kernel, dim3(grid), dim3(GA_THREADS), 0, st, a);
  return hipGetLastError();
}

}  // namespace lsa
