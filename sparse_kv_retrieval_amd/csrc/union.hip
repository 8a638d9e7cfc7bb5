// OR-mode union of the indexer layers' selections, compacted to an ascending
// index list ([BLOG] §4.2 of the FlashMemory-DeepSeek-V4 write-up: an entry is
// fetched if any of the layers predicts I >= 0.5; the hyper.ai digest,
// "方法", calls the fetched set C^MemComp).
//
// Grid: (chunk, sequence). A chunk is 256 mask words (16384 entries), one word
// per thread:
//  1. Each thread ORs its word over the layers and counts its bits. The
//     chunk's carry-in is the bit count of the sequence's earlier words, which
//     the block counts itself: thread t takes the earlier words t, t + 256, ...
//     and issues their loads together with those of its own word, so the whole
//     count costs one memory round trip for up to 8 earlier chunks. The kernel
//     needs no cross-block state and no scratch. The layer count is a template
//     parameter (rounded up to 1, 2, 3, 4 or 8; OR is idempotent, so the extra
//     slots re-read the last layer), which lets every load be unconditional and
//     in flight at once. One block scan of (earlier-word count, own count)
//     pairs gives the carry-in and every word's position.
//  2. Each wave then walks its 64 words in order. For word j it broadcasts the
//     word and its position, and every lane whose bit is set writes its entry
//     index at position + (set bits in the lanes below it) (mbcnt): one
//     coalesced store of consecutive indices per word.
#include "kernels.hpp"

namespace lsa {

static constexpr int UC_THREADS = 256;

template <int NL>
__global__ __launch_bounds__(UC_THREADS) void union_compact_kernel(const UnionArgs a) {
  constexpr int BATCH = NL <= 4 ? 8 : 4;  // earlier words per thread per round trip
  const int b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t w_lo = a.mwo[b], w_hi = a.mwo[b + 1];
  const int64_t row0 = a.key_off[b];
  const int64_t nb = a.key_off[b + 1] - row0;
  const int64_t nwords = w_hi - w_lo;
  const int64_t chunk0 = (int64_t)blockIdx.x * UC_THREADS;
  if (chunk0 >= nwords) {
    if (blockIdx.x == 0 && tid == 0) a.count_out[b] = 0;  // empty sequence
    return;
  }
  const uint64_t* m[NL];  // constant indices into the argument block: no dependent argument loads
  m[0] = a.mask[0] + w_lo;
#pragma unroll
  for (int l = 1; l < NL; ++l) m[l] = l < a.L ? a.mask[l] + w_lo : m[l - 1];

  // the thread's own word (a word past the end re-reads the chunk's first, and counts as 0)
  const int64_t wl = chunk0 + tid;
  const bool has = wl < nwords;
  const int64_t wr = has ? wl : chunk0;
  uint64_t own[NL];
#pragma unroll
  for (int l = 0; l < NL; ++l) own[l] = m[l][wr];

  // carry-in: the earlier words tid + 256 i, i < blockIdx.x (none of them is the last word)
  const int nbefore = (int)blockIdx.x;
  uint32_t before = 0;
  for (int i0 = 0; i0 < nbefore; i0 += BATCH) {
    uint64_t v[BATCH][NL];
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const int ii = i0 + i < nbefore ? i0 + i : nbefore - 1;
#pragma unroll
      for (int l = 0; l < NL; ++l) v[i][l] = m[l][tid + (int64_t)ii * UC_THREADS];
    }
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      uint64_t u = 0;
#pragma unroll
      for (int l = 0; l < NL; ++l) u |= v[i][l];
      before += i0 + i < nbefore ? (uint32_t)__popcll(u) : 0u;
    }
  }

  uint64_t u = 0;
#pragma unroll
  for (int l = 0; l < NL; ++l) u |= own[l];
  if (!has) u = 0;
  const int64_t first = wl * 64;
  if (has && first + 64 > nb) u &= (1ull << (nb - first)) - 1ull;  // bits past N_b (nb - first in [1, 63])
  if (has && a.union_out) a.union_out[w_lo + wl] = u;

  // one scan of (earlier-word count, own count): the carry-in is the total of the first halves
  int64_t tot;
  const int64_t ex = block_exclusive_scan(((int64_t)before << 32) | (int64_t)__popcll(u), &tot);
  const int64_t carry = tot >> 32;
  const uint32_t pos = (uint32_t)(carry + (ex & 0xFFFFFFFFll));  // < N_b < 2^31
  const int64_t chunk_total = tot & 0xFFFFFFFFll;

  // One word of the wave at a time (words past the end are 0): for word j, every lane whose bit
  // is set writes its entry index at the word's position + (set bits in the lanes below it): one
  // coalesced store of consecutive indices per word. Eight words at a time: their broadcasts
  // first, then eight buffer stores in which a lane without its bit stores out of range (the
  // store is dropped), so there is no branch and the stores overlap (with one wave per SIMD
  // there is little else to hide their latency).
  const auto ro = buf_rsrc(a.idx_out + row0, (uint32_t)nb * 4u);
  const int32_t wave_e0 = (int32_t)((wl - lane) * 64);  // the wave's first entry
  for (int j0 = 0; j0 < 64; j0 += 8) {
    uint32_t off[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t ulo = __builtin_amdgcn_readlane((uint32_t)u, j0 + i);
      const uint32_t uhi = __builtin_amdgcn_readlane((uint32_t)(u >> 32), j0 + i);
      const uint32_t pj = __builtin_amdgcn_readlane(pos, j0 + i);
      const uint32_t mine = lane < 32 ? (ulo >> lane) & 1u : (uhi >> (lane - 32)) & 1u;
      const uint32_t below = __builtin_amdgcn_mbcnt_hi(uhi, __builtin_amdgcn_mbcnt_lo(ulo, 0u));
      off[i] = mine ? (pj + below) * 4u : BUF_OOB;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_raw_buffer_store_b32((uint32_t)(wave_e0 + (j0 + i) * 64 + lane), ro, (int)off[i], 0, 0);
  }
  if (chunk0 + UC_THREADS >= nwords && tid == 0) a.count_out[b] = (int32_t)(carry + chunk_total);
}

hipError_t launch_union_compact(const UnionArgs& a, int B, int64_t max_words, hipStream_t st) {
  const int64_t chunks = max_words > 0 ? (max_words + UC_THREADS - 1) / UC_THREADS : 1;
  const dim3 grid((unsigned)chunks, (unsigned)B), block(UC_THREADS);
  switch (a.L) {
    case 1: hipLaunchKernelGGL(union_compact_kernel<1>, grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL(union_compact_kernel<2>, grid, block, 0, st, a); break;
    case 3: hipLaunchKernelGGL(union_compact_kernel<3>, grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL(union_compact_kernel<4>, grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL(union_compact_kernel<LSA_MAX_LAYERS>, grid, block, 0, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace lsa
