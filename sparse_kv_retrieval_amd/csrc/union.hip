// OR-mode union of the indexer layers' selections, compacted to an ascending
// index list ([BLOG] §4.2 of the FlashMemory-DeepSeek-V4 write-up: an entry is
// fetched if any of the layers predicts I >= 0.5; the hyper.ai digest,
// "方法", calls the fetched set C^MemComp).
//
// Grid: (chunk, sequence), 256 threads (four waves) per block. A chunk is 64 k
// mask words (k = 1..4, chosen by the launcher), 16 k per wave:
//  1. Lanes 0..16k-1 of wave v OR words 16k v + lane of the chunk over the
//     layers and count their bits, so thread order is word order. The chunk's
//     carry-in is the bit count of the sequence's earlier words, which the
//     block counts itself: thread t takes the earlier words t, t + 256, ...
//     and issues their loads together with those of its own word, so the
//     whole count costs one memory round trip for up to 2048 earlier words.
//     The kernel needs no cross-block state and no scratch. The layer count is
//     a template parameter (rounded up to 1, 2, 3, 4 or 8; OR is idempotent,
//     so the extra slots re-read the last layer), which lets every load be
//     unconditional and in flight at once. One block scan of (earlier-word
//     count, own count) pairs gives the carry-in and every word's position.
//  2. Each wave then walks its 16k words in order. For word j it broadcasts
//     the word and its position, and every lane whose bit is set writes its
//     entry index at position + (set bits in the lanes below it) (mbcnt): one
//     coalesced store of consecutive indices per word.
#include "kernels.hpp"

namespace lsa {

static constexpr int UC_THREADS = 256;

template <int NL>
__global__ __launch_bounds__(UC_THREADS) void union_compact_kernel(const UnionArgs a) {
  constexpr int BATCH = NL <= 4 ? 8 : 4;  // earlier words per thread per round trip
  const int b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t w_lo = a.mwo[b], w_hi = a.mwo[b + 1];
  const int64_t row0 = a.key_off[b];
  const int64_t nb = a.key_off[b + 1] - row0;
  const int64_t nwords = w_hi - w_lo;
  const int wpw = a.chunk_words / (UC_THREADS / 64);  // words per wave (16, 32, 48 or 64)
  const int64_t chunk0 = (int64_t)blockIdx.x * a.chunk_words;
  if (chunk0 >= nwords) {
    if (blockIdx.x == 0 && tid == 0) a.count_out[b] = 0;  // empty sequence
    return;
  }
  const uint64_t* m[NL];  // constant indices into the argument block: no dependent argument loads
  m[0] = a.mask[0] + w_lo;
#pragma unroll
  for (int l = 1; l < NL; ++l) m[l] = l < a.L ? a.mask[l] + w_lo : m[l - 1];

  // Own words: lanes 0..wpw-1 of wave v hold words v*wpw + lane of the chunk, so thread order
  // is word order for the block scan (the other lanes count 0). A word past the end re-reads
  // the chunk's first and counts as 0.
  const bool own_lane = lane < wpw;
  const int64_t wl = chunk0 + wv * wpw + (own_lane ? lane : 0);
  const bool has = own_lane && wl < nwords;
  const int64_t wr = has ? wl : chunk0;
  uint64_t own[NL];
#pragma unroll
  for (int l = 0; l < NL; ++l) own[l] = m[l][wr];

  // carry-in: the sequence's earlier words tid + UC_THREADS i, i < nbefore
  const int64_t nbw = chunk0;  // earlier words
  const int nbefore = (int)((nbw + UC_THREADS - 1) / UC_THREADS);
  uint32_t before = 0;
  for (int i0 = 0; i0 < nbefore; i0 += BATCH) {
    uint64_t v[BATCH][NL];
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const int64_t wi = tid + (int64_t)(i0 + i) * UC_THREADS;
      const int64_t wc = wi < nbw ? wi : 0;
#pragma unroll
      for (int l = 0; l < NL; ++l) v[i][l] = m[l][wc];
    }
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      uint64_t u = 0;
#pragma unroll
      for (int l = 0; l < NL; ++l) u |= v[i][l];
      before += tid + (int64_t)(i0 + i) * UC_THREADS < nbw ? (uint32_t)__popcll(u) : 0u;
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
  // store is dropped), so there is no branch and the stores overlap.
  const auto ro = buf_rsrc(a.idx_out + row0, (uint32_t)nb * 4u);
  const int32_t wave_e0 = (int32_t)((chunk0 + wv * wpw) * 64);  // the wave's first entry
  for (int j0 = 0; j0 < wpw; j0 += 8) {
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
  if (chunk0 + a.chunk_words >= nwords && tid == 0) a.count_out[b] = (int32_t)(carry + chunk_total);
}

hipError_t launch_union_compact(const UnionArgs& a, int B, int64_t max_words, int cus, hipStream_t st) {
  // Chunks of 64 k words (16 k per wave), k = 1..4: the smallest k for which the grid is at most
  // one block per compute unit, so a short list of sequences still spreads over the device
  // (each wave then walks fewer words), while many or long sequences keep their blocks few
  // (every block re-reads its sequence's earlier words).
  UnionArgs c = a;
  int k = 1;
  while (k < 4 && (max_words + 64 * k - 1) / (64 * k) * (int64_t)B > (int64_t)cus) ++k;
  c.chunk_words = 64 * k;
  const int64_t chunks = max_words > 0 ? (max_words + c.chunk_words - 1) / c.chunk_words : 1;
  const dim3 grid((unsigned)chunks, (unsigned)B), block(UC_THREADS);
  switch (c.L) {
    case 1: hipLaunchKernelGGL(union_compact_kernel<1>, grid, block, 0, st, c); break;
    case 2: hipLaunchKernelGGL(union_compact_kernel<2>, grid, block, 0, st, c); break;
    case 3: hipLaunchKernelGGL(union_compact_kernel<3>, grid, block, 0, st, c); break;
    case 4: hipLaunchKernelGGL(union_compact_kernel<4>, grid, block, 0, st, c); break;
    default: hipLaunchKernelGGL(union_compact_kernel<LSA_MAX_LAYERS>, grid, block, 0, st, c); break;
  }
  return hipGetLastError();
}

}  // namespace lsa
