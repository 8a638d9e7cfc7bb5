// OR-mode union of the indexer layers' selections, compacted to an ascending
// index list ([BLOG] §4.2 of the FlashMemory-DeepSeek-V4 write-up: an entry is
// fetched if any of the layers predicts I >= 0.5; the hyper.ai digest,
// "方法", calls the fetched set C^MemComp).
//
// Grid: (chunk, sequence). A chunk is 256 mask words (16384 entries), one word
// per thread:
//  1. Each thread ORs its word over the layers and counts its bits. The
//     chunk's carry-in is the bit count of the sequence's earlier words, which
//     the block counts itself in one strided pass (its loads issued four words
//     at a time, so the pass costs about one memory round trip per 1024
//     earlier words): the kernel needs no cross-block state and no scratch.
//     One block scan of (earlier-word count, own count) pairs gives the
//     carry-in and every word's position.
//  2. Each wave then walks its 64 words in order. For word j it broadcasts the
//     word and its position, and every lane whose bit is set writes its entry
//     index at position + (set bits in the lanes below it) (mbcnt): one
//     coalesced store of consecutive indices per word.
#include "kernels.hpp"

namespace lsa {

static constexpr int UC_THREADS = 256;

__global__ __launch_bounds__(UC_THREADS) void union_compact_kernel(const UnionArgs a) {
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int64_t w_lo = a.mwo[b], w_hi = a.mwo[b + 1];
  const int64_t nwords = w_hi - w_lo;
  const int64_t chunk0 = (int64_t)blockIdx.x * UC_THREADS;
  if (chunk0 >= nwords) {
    if (blockIdx.x == 0 && threadIdx.x == 0) a.count_out[b] = 0;  // empty sequence
    return;
  }
  const int64_t row0 = a.key_off[b];
  const int64_t nb = a.key_off[b + 1] - row0;

  // OR over the layers of word wl of the sequence (no tail masking)
  auto load_or = [&](int64_t wl) -> uint64_t {
    uint64_t u = 0;
#pragma unroll
    for (int l = 0; l < LSA_MAX_LAYERS; ++l)
      if (l < a.L) u |= a.mask[l][w_lo + wl];
    return u;
  };

  // carry-in: union bits of the earlier words of this sequence (none of them is the last word)
  uint32_t before = 0;
  int64_t wp = threadIdx.x;
  for (; wp + 3 * UC_THREADS < chunk0; wp += 4 * UC_THREADS) {
    const uint64_t u0 = load_or(wp), u1 = load_or(wp + UC_THREADS);
    const uint64_t u2 = load_or(wp + 2 * UC_THREADS), u3 = load_or(wp + 3 * UC_THREADS);
    before += __popcll(u0) + __popcll(u1) + __popcll(u2) + __popcll(u3);
  }
  for (; wp < chunk0; wp += UC_THREADS) before += __popcll(load_or(wp));

  const int64_t wl = chunk0 + threadIdx.x;
  const bool has = wl < nwords;
  uint64_t u = has ? load_or(wl) : 0ull;
  const int64_t first = wl * 64;
  if (has && first + 64 > nb) u &= (1ull << (nb - first)) - 1ull;  // bits past N_b (nb - first in [1, 63])
  if (has && a.union_out) a.union_out[w_lo + wl] = u;

  // one scan of (earlier-word count, own count): the carry-in is the total of the first halves
  int64_t tot;
  const int64_t ex = block_exclusive_scan(((int64_t)before << 32) | (int64_t)__popcll(u), &tot);
  const int64_t carry = tot >> 32;
  const int64_t pos = carry + (ex & 0xFFFFFFFFll);
  const int64_t chunk_total = tot & 0xFFFFFFFFll;

  // coalesced writes, one word of the wave at a time (words past the end are 0)
  int32_t* out = a.idx_out + row0;
  const int64_t wave_w0 = wl - lane;  // the wave's first word
#pragma unroll 4
  for (int j = 0; j < 64; ++j) {
    const uint32_t ulo = __builtin_amdgcn_readlane((uint32_t)u, j);
    const uint32_t uhi = __builtin_amdgcn_readlane((uint32_t)(u >> 32), j);
    if ((ulo | uhi) == 0u) continue;  // uniform
    const uint32_t plo = __builtin_amdgcn_readlane((uint32_t)pos, j);
    const uint32_t phi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)pos >> 32), j);
    const int64_t pj = (int64_t)(((uint64_t)phi << 32) | plo);
    const uint64_t word = ((uint64_t)uhi << 32) | ulo;
    if ((word >> lane) & 1ull) {
      const uint32_t below = __builtin_amdgcn_mbcnt_hi(uhi, __builtin_amdgcn_mbcnt_lo(ulo, 0u));
      out[pj + below] = (int32_t)((wave_w0 + j) * 64 + lane);
    }
  }
  if (chunk0 + UC_THREADS >= nwords && threadIdx.x == 0) a.count_out[b] = (int32_t)(carry + chunk_total);
}

hipError_t launch_union_compact(const UnionArgs& a, int B, int64_t max_words, hipStream_t st) {
  const int64_t chunks = max_words > 0 ? (max_words + UC_THREADS - 1) / UC_THREADS : 1;
  hipLaunchKernelGGL(union_compact_kernel, dim3((unsigned)chunks, (unsigned)B), dim3(UC_THREADS), 0, st, a);
  return hipGetLastError();
}

}  // namespace lsa
