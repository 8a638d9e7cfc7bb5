// OR-mode union of the indexer layers' selections, compacted to an ascending
// index list ([BLOG] §4.2 of the FlashMemory-DeepSeek-V4 write-up: an entry is
// fetched if any of the layers predicts I >= 0.5; the hyper.ai digest,
// "方法", calls the fetched set C^MemComp).
//
// Grid: (chunk, sequence). A chunk is 256 mask words (16384 entries), one word
// per thread. Each thread ORs its word over the layers and counts the bits.
// A block scan gives each word's output position within the chunk. The
// chunk's base position is the number of union bits in all earlier words of
// the sequence, which the block re-counts itself (at most a few thousand
// words). That keeps the kernel free of cross-block state and scratch memory.
#include "kernels.hpp"

namespace lsa {

static constexpr int UC_THREADS = 256;

__global__ __launch_bounds__(UC_THREADS) void union_compact_kernel(const UnionArgs a) {
  const int b = blockIdx.y;
  const int64_t w_lo = a.mwo[b], w_hi = a.mwo[b + 1];
  const int64_t nwords = w_hi - w_lo;
  const int64_t chunk0 = (int64_t)blockIdx.x * UC_THREADS;
  if (chunk0 >= nwords) {
    if (blockIdx.x == 0 && threadIdx.x == 0) a.count_out[b] = 0;  // empty sequence
    return;
  }
  const int64_t row0 = a.key_off[b];
  const int64_t nb = a.key_off[b + 1] - row0;

  auto load_union = [&](int64_t wl) -> uint64_t {
    uint64_t u = 0;
    for (int l = 0; l < a.L; ++l) u |= a.mask[l][w_lo + wl];
    const int64_t first = wl * 64;
    if (first + 64 > nb) u &= (nb - first >= 64) ? ~0ull : ((1ull << (nb - first)) - 1ull);
    return u;
  };

  // carry-in: union bits in words [0, chunk0) of this sequence
  int64_t before = 0;
  for (int64_t wl = threadIdx.x; wl < chunk0; wl += UC_THREADS) before += __popcll(load_union(wl));
  int64_t carry;
  (void)block_exclusive_scan(before, &carry);

  const int64_t wl = chunk0 + threadIdx.x;
  const bool has = wl < nwords;
  const uint64_t u = has ? load_union(wl) : 0ull;
  if (has && a.union_out) a.union_out[w_lo + wl] = u;
  int64_t chunk_total;
  const int64_t pos = carry + block_exclusive_scan(__popcll(u), &chunk_total);

  int32_t* out = a.idx_out + row0 + pos;
  uint64_t bits = u;
  const int32_t sbase = (int32_t)(wl * 64);
  for (int j = 0; bits; ++j) {
    const int bit = __builtin_ctzll(bits);
    out[j] = sbase + bit;
    bits &= bits - 1;
  }
  if (chunk0 + UC_THREADS >= nwords && threadIdx.x == 0) a.count_out[b] = (int32_t)(carry + chunk_total);
}

hipError_t launch_union_compact(const UnionArgs& a, int B, int64_t max_words, hipStream_t st) {
  const int64_t chunks = max_words > 0 ? (max_words + UC_THREADS - 1) / UC_THREADS : 1;
  hipLaunchKernelGGL(union_compact_kernel, dim3((unsigned)chunks, (unsigned)B), dim3(UC_THREADS), 0, st, a);
  return hipGetLastError();
}

}  // namespace lsa
