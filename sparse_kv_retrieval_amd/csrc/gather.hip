// Load step: copy the selected compressed-KV rows into a compact buffer (the
// hyper.ai digest of FlashMemory-DeepSeek-V4, "方法": C^MemComp is loaded into
// GPU memory). The pool is either in HBM (lsa_gather) or in pinned host
// memory (lsa_fetch_host: the cold pool of the write-up, read over the host
// link without a staging copy); the kernel is the same, with more rows in
// flight per wave for the host link's longer latency.
//
// Each block computes, in LDS, where every sequence's rows land: a prefix sum
// of min(count, capacity) in explicit mode, or of count in packed mode. For up
// to GA_TAB sequences it also keeps the per-sequence pool, list and output
// offsets in LDS. The output rows are numbered 0..total-1, and each wave moves
// GA_ROWS consecutive ones per iteration. Lanes 0..GA_ROWS-1 resolve one row
// each (sequence, source row, destination row) and broadcast it, so a row costs
// one dependent global load (its list entry) before the copy. The copy itself
// issues all the rows' 16-byte non-temporal loads before their stores, so each
// 1 KiB latent row is one fully coalesced wave access and GA_ROWS KiB per wave
// are in flight.
#include "kernels.hpp"

namespace lsa {

static constexpr int GA_THREADS = 256;

#if LSA_DEBUG_CHECKS
static __device__ unsigned int g_gather_range_errors;
#endif
static constexpr int GA_TAB = 1024;  // sequences whose offsets are cached in LDS

// Dynamic LDS: pre[B+1], then (for B <= GA_TAB) t_pool[B], t_idx[B], t_out[B], all int64.
// GA_ROWS rows per wave per iteration (at most 64: one lane resolves each).
template <int GA_ROWS>
__global__ __launch_bounds__(GA_THREADS) void gather_kernel(const GatherArgs a) {
  static_assert(GA_ROWS >= 1 && GA_ROWS <= 64, "rows per wave");
  extern __shared__ int64_t dyn[];
  const bool cached = a.B <= GA_TAB;
  int64_t* pre = dyn;
  int64_t* t_pool = dyn + a.B + 1;
  int64_t* t_idx = t_pool + a.B;
  int64_t* t_out = t_idx + a.B;
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
    if (cached) {
      for (int b = tid; b < a.B; b += GA_THREADS) {
        t_pool[b] = a.pool_off[b];
        t_idx[b] = a.idx_off[b];
        t_out[b] = a.out_off ? a.out_off[b] : 0;
      }
    }
    __syncthreads();
  }
  const int64_t total = pre[a.B];
  const int lane = tid & 63;
  const int wave_in_block = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t nw = (int64_t)gridDim.x * (GA_THREADS / 64);
  const int n16 = (int)(a.row_bytes >> 4);
  for (int64_t r0 = ((int64_t)blockIdx.x * (GA_THREADS / 64) + wave_in_block) * GA_ROWS; r0 < total;
       r0 += nw * GA_ROWS) {
    // lane u < GA_ROWS resolves output row r0 + u
    int64_t src_row = 0, dst_row = 0;
    int ok = 0;
    if (lane < GA_ROWS) {
      const int64_t r = r0 + lane;
      if (r < total) {
        const int b = upper_seq(pre, a.B, r);
        const int64_t i = r - pre[b];
        const int64_t po = cached ? t_pool[b] : a.pool_off[b];
        const int64_t io = cached ? t_idx[b] : a.idx_off[b];
        dst_row = a.out_off ? (cached ? t_out[b] : a.out_off[b]) + i : r;
        ok = dst_row < a.out_capacity;
        const int32_t e = a.idx[io + i];
        src_row = po + e;
#if LSA_DEBUG_CHECKS
        if (ok && (e < 0 || e >= a.pool_off[b + 1] - po)) {
          atomicAdd(&g_gather_range_errors, 1u);
          ok = 0;
        }
#endif
      }
    }
    const char* src[GA_ROWS];
    char* dst[GA_ROWS];
    bool okr[GA_ROWS];
#pragma unroll
    for (int u = 0; u < GA_ROWS; ++u) {
      okr[u] = __shfl(ok, u) != 0;
      src[u] = a.pool + (int64_t)__shfl(src_row, u) * a.row_bytes;
      dst[u] = a.out + (int64_t)__shfl(dst_row, u) * a.row_bytes;
    }
    for (int j = lane; j < n16; j += 64) {
      u32x4 v[GA_ROWS];
#pragma unroll
      for (int u = 0; u < GA_ROWS; ++u)
        if (okr[u]) v[u] = __builtin_nontemporal_load((const u32x4*)src[u] + j);
#pragma unroll
      for (int u = 0; u < GA_ROWS; ++u)
        if (okr[u]) __builtin_nontemporal_store(v[u], (u32x4*)dst[u] + j);
    }
  }
}

hipError_t gather_take_range_errors(unsigned int* out) {
#if LSA_DEBUG_CHECKS
  hipError_t e = hipMemcpyFromSymbol(out, HIP_SYMBOL(g_gather_range_errors), sizeof(unsigned int));
  if (e != hipSuccess) return e;
  const unsigned int zero = 0;
  return hipMemcpyToSymbol(HIP_SYMBOL(g_gather_range_errors), &zero, sizeof(unsigned int));
#else
  *out = 0;
  return hipSuccess;
#endif
}

hipError_t launch_gather(const GatherArgs& a, int grid, int rows_per_wave, hipStream_t st) {
  const size_t lds = sizeof(int64_t) * ((size_t)a.B + 1 + (a.B <= GA_TAB ? 3 * (size_t)a.B : 0));
  switch (rows_per_wave) {
    case 16: hipLaunchKernelGGL(gather_kernel<16>, dim3(grid), dim3(GA_THREADS), lds, st, a); break;
    case 32: hipLaunchKernelGGL(gather_kernel<32>, dim3(grid), dim3(GA_THREADS), lds, st, a); break;
    default: hipLaunchKernelGGL(gather_kernel<8>, dim3(grid), dim3(GA_THREADS), lds, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace lsa
