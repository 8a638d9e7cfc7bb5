// Top-k inside the loaded subset: the second level of the two-level selection
// ([BLOG] §3.2 of the FlashMemory-DeepSeek-V4 write-up: the native Lightning
// Indexer picks the final top-k core entries inside C^MemComp).
//
// One block per (sequence, layer). The scores y are in the workspace, in
// subset order, which is ascending entry order, with a histogram of their top
// 11 key bits that the scoring kernel built. A radix select over
// order-preserving uint32 keys finds T, the key of the k-th largest score, and
// how many entries equal to T must be kept. The output keeps every entry above
// T plus the lowest-index entries equal to it, in list order, which matches
// the (-y, s) order and keeps the output ascending.
#include "kernels.hpp"

namespace lsa {

static constexpr int TS_THREADS = 1024;
static constexpr int TS_VMAX = 32;  // values per thread held in registers (lists up to 32,768)
static constexpr int TS_RMAX = 128; // values per thread of the reloading select (lists up to 131,072)
static constexpr int TS_RC = 16;    // values per thread per round trip of the reloading select
static_assert((int64_t)TS_THREADS * TS_RMAX == TOPK_NOHIST_MAX_ROWS, "lists without the scorer's histogram");

// Number of set bits of m in the lanes below this one.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Block-wide exclusive prefix of small per-thread values v < 2^NBITS, and the
// block total. Within a wave the prefix is bit-sliced: one ballot per bit and
// a count of the lanes below (no shuffles, no LDS). The 16 wave totals go
// through LDS. Costs two barriers; `wt` is a 16-entry LDS scratch table.
template <int NBITS>
__device__ __forceinline__ uint32_t block_prefix_small(uint32_t v, uint32_t* wt, uint32_t& total) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int b = 0; b < NBITS; ++b) {
    const uint64_t m = __ballot((v >> b) & 1u);
    pre += lanes_below(m) << b;
    tot += (uint32_t)__popcll(m) << b;
  }
  if (lane == 0) wt[w] = tot;
  __syncthreads();
  uint32_t off = 0, all = 0;
#pragma unroll
  for (int i = 0; i < TS_THREADS / 64; ++i) {
    const uint32_t x = wt[i];
    off += i < w ? x : 0u;
    all += x;
  }
  __syncthreads();
  total = all;
  return off + pre;
}

// Block-wide exclusive prefix of 32-bit values (wave scan by shuffles, then
// the wave totals through LDS), and the block total. Two barriers.
__device__ __forceinline__ uint32_t block_prefix_u32(uint32_t v, uint32_t* wt, uint32_t& total) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wt[w] = x;
  __syncthreads();
  uint32_t off = 0, all = 0;
#pragma unroll
  for (int i = 0; i < TS_THREADS / 64; ++i) {
    const uint32_t t = wt[i];
    off += i < w ? t : 0u;
    all += t;
  }
  __syncthreads();
  total = all;
  return off + x - v;
}

// The digit d with (count of digits > d) < krem <= (count of digits >= d),
// over an LDS histogram of nbins (1024 or 2048) bins. It writes d and the
// new krem (how many of the entries with digit d are still to be taken).
__device__ __forceinline__ void find_digit(const uint32_t* hist, int nbins, uint32_t krem, uint32_t* sh_digit,
                                           uint32_t* sh_krem) {
  const int tid = threadIdx.x;
  const int per = nbins / TS_THREADS;
  __shared__ uint32_t wt[TS_THREADS / 64];
  uint32_t own = 0;
  for (int i = 0; i < per; ++i) own += hist[tid * per + i];
  uint32_t tot;
  const uint32_t below = block_prefix_u32(own, wt, tot);  // bins below this thread's bins
  const uint32_t suf = tot - below;                        // bins >= tid*per
  const uint32_t above = suf - own;                        // bins above this thread's bins
  if (above < krem && krem <= suf) {
    uint32_t cum = above;
    for (int i = per - 1; i >= 0; --i) {
      const uint32_t c = hist[tid * per + i];
      if (cum + c >= krem) {
        *sh_digit = (uint32_t)(tid * per + i);
        *sh_krem = krem - cum;
        break;
      }
      cum += c;
    }
  }
  __syncthreads();
}

// Radix select over a list held in registers.
//
// Thread t = 64 w + lane holds the list entries i = t + 1024 v (v < V), so
// every load is coalesced; all of a thread's loads (and its share of the
// histogram) are issued before any is used, so the list costs one memory round
// trip. The list order is (v, w, lane): an entry's rank among the entries
// before it is a count of lanes below it in its wave (ballot + mbcnt) plus an
// exclusive scan of per-(v, w) counts held in a small LDS table.
//
// T, the key of the k-th largest score, comes from the scoring kernel's
// histogram (hist_bl, the 2048 counts of the list's keys by their top 11
// bits): it gives the bin d of the k-th largest key and its rank inside the
// bin; the keys of bin d are appended to an LDS list (one LDS atomic per wave);
// and one wave finds T among them bit by bit (no barrier), or, for a crowded
// bin, the block runs the last two radix levels on that list. Without a usable
// histogram, three histogram passes over bits 31..21, 20..10 and 9..0 of the
// keys find T.
//
// The output keeps every key above T and the first krem keys equal to T in
// list order, which settles ties toward the lower index. One scan of the
// per-(v, w) counts of keys above T and keys equal to T places them all: the
// taken entries before an entry number (above before) + min(equal before,
// krem). The list's entry indices are loaded with the scores, so each thread
// stores its taken entries (index and score) straight from registers.
__device__ __forceinline__ void lds_select(const uint32_t* keys, int n, uint32_t rank, uint32_t* hist,
                                           uint32_t* sh_digit, uint32_t* sh_krem, uint32_t& T, uint32_t& krem,
                                           int passes, int first_pass, uint32_t prefix);
static constexpr int TS_CCAP = 4096;  // keys of the k-th bin held in LDS
static constexpr int TS_WCAP = 512;   // at most this many: one wave finds T
static constexpr int TS_OCAP = 4096;  // outputs placed through LDS

// LDS of the in-register select (one copy per block, whichever list length is instantiated)
struct RegSelectSmem {
  uint32_t hist[2048];
  uint32_t tab[TS_RMAX * (TS_THREADS / 64)], tab2[TS_RMAX * (TS_THREADS / 64)];
  uint32_t cand[TS_CCAP];
  int32_t osrc[TS_OCAP];
  uint64_t bal[2][TS_RMAX * (TS_THREADS / 64)];  // the reloading select: ballots of keys above and equal to T
  int32_t cpos[TS_CCAP];                          // the reloading select: list positions of the candidates
  uint32_t wt[2][TS_THREADS / 64];
  uint32_t sh_digit, sh_krem, ncand;
};

// Exclusive scan, in place, of two LDS tables of n <= 2 * TS_THREADS counts each (counts <= 64).
__device__ __forceinline__ void table_exclusive_scan2(uint32_t* ta, uint32_t* te, int n, uint32_t (&wt)[2][16]) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int j0 = 2 * tid;
  const uint32_t a0 = j0 < n ? ta[j0] : 0u, a1 = j0 + 1 < n ? ta[j0 + 1] : 0u;
  const uint32_t e0 = j0 < n ? te[j0] : 0u, e1 = j0 + 1 < n ? te[j0 + 1] : 0u;
  // both prefixes bit-sliced at once: per-thread sums are at most 128 (8 bits)
  const uint32_t va = a0 + a1, ve = e0 + e1;
  uint32_t pa = 0, pe = 0, sa = 0, se = 0;
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const uint64_t ma = __ballot((va >> b) & 1u), me = __ballot((ve >> b) & 1u);
    pa += lanes_below(ma) << b;
    pe += lanes_below(me) << b;
    sa += (uint32_t)__popcll(ma) << b;
    se += (uint32_t)__popcll(me) << b;
  }
  if (lane == 0) {
    wt[0][w] = sa;
    wt[1][w] = se;
  }
  __syncthreads();
  uint32_t oa = 0, oe = 0;
#pragma unroll
  for (int i = 0; i < TS_THREADS / 64; ++i) {
    oa += i < w ? wt[0][i] : 0u;
    oe += i < w ? wt[1][i] : 0u;
  }
  if (j0 < n) {
    ta[j0] = oa + pa;
    te[j0] = oe + pe;
  }
  if (j0 + 1 < n) {
    ta[j0 + 1] = oa + pa + a0;
    te[j0 + 1] = oe + pe + e0;
  }
  __syncthreads();
}

// VM: values per thread held in registers (the list has at most TS_THREADS * VM entries).
template <int VM>
__device__ __forceinline__ void select_in_registers(const float* __restrict__ ys, const int32_t* __restrict__ idx,
                                                    int32_t M, int32_t k, int32_t* out, float* outs,
                                                    const uint32_t* __restrict__ hist_bl, RegSelectSmem& sm) {
  static_assert(VM % 8 == 0 && VM <= TS_VMAX, "values per thread");
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  constexpr int NW = TS_THREADS / 64;
  const int V = (M + TS_THREADS - 1) / TS_THREADS;
  // Key 0 pads the tail. It sorts below every real key (the smallest real key,
  // -inf, maps to 0x007FFFFF), so padding never reaches the selected bins or
  // the output, and the passes need no bounds test. Every load is issued first
  // (clamped addresses, no branch), then the keys are formed.
  // Lists of up to 32 values per thread load in one round trip; longer ones in round trips of 16.
  // The entry indices of the list come in the same round trip, so the taken entries are stored
  // straight from registers at the end.
  constexpr int LC = VM <= 32 ? VM : 16;
  uint32_t key[VM];
  int32_t ent[VM];
  uint32_t hv[2048 / TS_THREADS];
#pragma unroll
  for (int u = 0; u < 2048 / TS_THREADS; ++u) hv[u] = hist_bl ? hist_bl[tid + TS_THREADS * u] : 0u;
#pragma unroll
  for (int c = 0; c < VM; c += LC) {
    if (c < V) {
#pragma unroll
      for (int v = c; v < c + LC; ++v) {
        key[v] = __float_as_uint(ys[min(tid + TS_THREADS * v, M - 1)]);
        ent[v] = idx[min(tid + TS_THREADS * v, M - 1)];
      }
#pragma unroll
      for (int v = c; v < c + LC; ++v)
        key[v] = (v < V && tid + TS_THREADS * v < M) ? order_key(__uint_as_float(key[v])) : 0u;
    }
  }

  uint32_t* hist = sm.hist;
  uint32_t* tab = sm.tab;
  uint32_t* tab2 = sm.tab2;
  uint32_t* cand = sm.cand;
  uint32_t& sh_digit = sm.sh_digit;
  uint32_t& sh_krem = sm.sh_krem;
  uint32_t& ncand = sm.ncand;
  uint32_t prefix = 0, pmask = 0, krem = (uint32_t)k;
  bool found = false;
  if (hist_bl) {
#pragma unroll
    for (int u = 0; u < 2048 / TS_THREADS; ++u) hist[tid + TS_THREADS * u] = hv[u];
    if (tid == 0) ncand = 0;
    __syncthreads();
    find_digit(hist, 2048, (uint32_t)k, &sh_digit, &sh_krem);
    const uint32_t d = sh_digit, bin_rank = sh_krem, nd = hist[d];
    if (nd <= (uint32_t)TS_CCAP) {  // uniform
      // the keys of bin d, in any order: one LDS atomic per wave reserves the wave's run
      uint32_t wc = 0;
#pragma unroll
      for (int v = 0; v < VM; ++v)
        if (v < V) wc += (uint32_t)__popcll(__ballot((key[v] >> 21) == d && key[v] != 0u));
      uint32_t base = 0;
      if (lane == 0 && wc) base = atomicAdd(&ncand, wc);
      base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
      for (int v = 0; v < VM; ++v)
        if (v < V) {
          const bool in = (key[v] >> 21) == d && key[v] != 0u;
          const uint64_t m = __ballot(in);
          if (in) cand[base + lanes_below(m)] = key[v];
          base += (uint32_t)__popcll(m);
        }
      __syncthreads();
      const uint32_t nc = ncand;
      if (nc <= (uint32_t)TS_WCAP) {
        if (w == 0) {
          // the bin_rank-th largest of the nc keys, bit by bit below the bin's 11 bits
          uint32_t kk[TS_WCAP / 64];
#pragma unroll
          for (int u = 0; u < TS_WCAP / 64; ++u) {
            const uint32_t j = 64u * u + lane;
            kk[u] = j < nc ? cand[j] : 0u;  // key 0 ranks below every value tried
          }
          uint32_t t = d << 21;
          for (int b = 20; b >= 0; --b) {
            const uint32_t c = t | (1u << b);
            uint32_t cnt = 0;
#pragma unroll
            for (int u = 0; u < TS_WCAP / 64; ++u) cnt += (uint32_t)__popcll(__ballot(kk[u] >= c));
            if (cnt >= bin_rank) t = c;
          }
          uint32_t gt = 0;
#pragma unroll
          for (int u = 0; u < TS_WCAP / 64; ++u) gt += (uint32_t)__popcll(__ballot(kk[u] > t));
          if (lane == 0) {
            sh_digit = t;
            sh_krem = bin_rank - gt;
          }
        }
        __syncthreads();
        prefix = sh_digit;
        krem = sh_krem;
      } else {
        uint32_t Tb, kb;
        lds_select(cand, (int)nc, bin_rank, hist, &sh_digit, &sh_krem, Tb, kb, 3, 1, d << 21);
        prefix = Tb;
        krem = kb;
      }
      found = true;
    }
    __syncthreads();
  }
#pragma unroll
  for (int pass = 0; pass < (found ? 0 : 3); ++pass) {
    const int sh = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nb = pass == 2 ? 1024 : 2048;
    for (int i = tid; i < 2048; i += TS_THREADS) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int v = 0; v < VM; ++v)
      if (v < V && (key[v] & pmask) == prefix) atomicAdd(&hist[(key[v] >> sh) & (nb - 1)], 1u);
    __syncthreads();
    find_digit(hist, nb, krem, &sh_digit, &sh_krem);
    prefix |= sh_digit << sh;
    pmask |= (uint32_t)(nb - 1) << sh;
    krem = sh_krem;
    __syncthreads();
  }
  const uint32_t T = prefix;

  // tab: per-(v, w) counts of keys above T, tab2: of keys equal to T; then one scan of both.
  // (Ballots are recomputed in each loop rather than kept, so registers hold only the keys.)
#pragma unroll
  for (int v = 0; v < VM; ++v)
    if (v < V) {
      const uint64_t ma = __ballot(key[v] > T), me = __ballot(key[v] == T);
      if (lane == 0) {
        tab[v * NW + w] = (uint32_t)__popcll(ma);
        tab2[v * NW + w] = (uint32_t)__popcll(me);
      }
    }
  __syncthreads();
  table_exclusive_scan2(tab, tab2, V * NW, sm.wt);
  // output position of entry (v, w, lane) if it is taken, else -1
  auto place = [&](int v) -> int32_t {
    const uint64_t ma = __ballot(key[v] > T), me = __ballot(key[v] == T);
    const uint32_t ab = tab[v * NW + w] + lanes_below(ma), eb = tab2[v * NW + w] + lanes_below(me);
    const bool take = key[v] > T || (key[v] == T && eb < krem);
    return take ? (int32_t)(ab + min(eb, krem)) : -1;
  };
  // every taken entry straight from registers: its index, and its score (the inverse of order_key)
#pragma unroll
  for (int v = 0; v < VM; ++v)
    if (v < V) {
      const int32_t pos = place(v);
      if (pos >= 0 && pos < k) {  // exactly k are taken; the bound only guards a mismatched workspace
        out[pos] = ent[v];
        if (outs) {
          const uint32_t kv = key[v];
          outs[pos] = __uint_as_float((kv & 0x80000000u) ? (kv & 0x7FFFFFFFu) : ~kv);
        }
      }
    }
}

// Lists longer than the in-register select holds (up to TS_THREADS x TS_RMAX
// entries): the same steps, with the scores read again from memory, TS_RC per
// thread at a time, wherever the keys are needed, instead of held in
// registers. Thread t handles entries t + TS_THREADS v as before. The pass
// that collects the candidates (the keys that share the k-th key's prefix)
// also keeps, in LDS, the ballots of the keys with a higher prefix, which are
// all taken; once T is known the candidates above and equal to T set their own
// bits from their list positions, so no further read is needed. When the histogram bin of the k-th key holds more than
// TS_CCAP keys, one more read counts their next 11 bits and narrows the
// candidates to a 22-bit prefix. Returns false, having written nothing, when
// even that prefix is shared by more than TS_CCAP keys (massive ties); the
// caller then runs the streaming select.
__device__ __forceinline__ void reload_keys(const float* __restrict__ ys, int32_t M, int c, int V,
                                            uint32_t (&kv)[TS_RC]) {
  const int tid = threadIdx.x;
  float y[TS_RC];
#pragma unroll
  for (int u = 0; u < TS_RC; ++u) y[u] = ys[min(tid + TS_THREADS * (c + u), M - 1)];
#pragma unroll
  for (int u = 0; u < TS_RC; ++u)
    kv[u] = (c + u < V && tid + TS_THREADS * (c + u) < M) ? order_key(y[u]) : 0u;
}

__device__ __forceinline__ bool select_reload(const float* __restrict__ ys, const int32_t* __restrict__ idx,
                                              int32_t M, int32_t k, int32_t* out, float* outs,
                                              const uint32_t* __restrict__ hist_bl, RegSelectSmem& sm) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  constexpr int NW = TS_THREADS / 64;
  const int V = (M + TS_THREADS - 1) / TS_THREADS;
  if (hist_bl) {
    for (int i = tid; i < 2048; i += TS_THREADS) sm.hist[i] = hist_bl[i];
  } else {
    // no histogram from the scorer: count the keys' top 11 bits in one more read of the list
    for (int i = tid; i < 2048; i += TS_THREADS) sm.hist[i] = 0u;
    __syncthreads();
    for (int c = 0; c < TS_RMAX; c += TS_RC) {
      if (c >= V) break;  // uniform
      uint32_t kv[TS_RC];
      reload_keys(ys, M, c, V, kv);
#pragma unroll
      for (int u = 0; u < TS_RC; ++u)
        if (kv[u] != 0u) atomicAdd(&sm.hist[kv[u] >> 21], 1u);
    }
  }
  if (tid == 0) sm.ncand = 0;
  __syncthreads();
  find_digit(sm.hist, 2048, (uint32_t)k, &sm.sh_digit, &sm.sh_krem);
  const uint32_t d = sm.sh_digit, nd = sm.hist[d];
  // the k-th key has the top bits `pre` (under `pmask`) and is the rank-th largest of the keys that do
  uint32_t pre = d << 21, pmask = 0xFFE00000u, rank = sm.sh_krem;
  int low = 21;  // bits below the known prefix
  __syncthreads();
  if (nd > (uint32_t)TS_CCAP) {  // uniform
    // a crowded bin: one more level, the counts of bits 20..10 of the bin's keys
    for (int i = tid; i < 2048; i += TS_THREADS) sm.hist[i] = 0u;
    __syncthreads();
    for (int c = 0; c < TS_RMAX; c += TS_RC) {
      if (c >= V) break;  // uniform
      uint32_t kv[TS_RC];
      reload_keys(ys, M, c, V, kv);
#pragma unroll
      for (int u = 0; u < TS_RC; ++u)
        if ((kv[u] & pmask) == pre && kv[u] != 0u) atomicAdd(&sm.hist[(kv[u] >> 10) & 2047u], 1u);
    }
    __syncthreads();
    find_digit(sm.hist, 2048, rank, &sm.sh_digit, &sm.sh_krem);
    const uint32_t d2 = sm.sh_digit, n2 = sm.hist[d2];
    rank = sm.sh_krem;
    __syncthreads();
    if (n2 > (uint32_t)TS_CCAP) return false;  // uniform: massive ties
    pre |= d2 << 10;
    pmask = 0xFFFFFC00u;
    low = 10;
  }

  // the keys with the prefix, in any order: one LDS atomic per wave and round trip reserves the
  // wave's run (one per value would serialise on the shared counter)
  for (int c = 0; c < TS_RMAX; c += TS_RC) {
    if (c >= V) break;  // uniform
    uint32_t kv[TS_RC];
    reload_keys(ys, M, c, V, kv);
    uint32_t wc = 0;
#pragma unroll
    for (int u = 0; u < TS_RC; ++u) wc += (uint32_t)__popcll(__ballot((kv[u] & pmask) == pre && kv[u] != 0u));
    uint32_t base = 0;
    if (lane == 0 && wc) base = atomicAdd(&sm.ncand, wc);
    base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
    for (int u = 0; u < TS_RC; ++u) {
      const bool in = (kv[u] & pmask) == pre && kv[u] != 0u;
      const uint64_t m = __ballot(in);
      const uint32_t j = base + lanes_below(m);
      if (in && j < (uint32_t)TS_CCAP) {  // (bounded: a histogram that does not match the scores)
        sm.cand[j] = kv[u];
        sm.cpos[j] = tid + TS_THREADS * (c + u);
      }
      base += (uint32_t)__popcll(m);
      // keys whose prefix is above the k-th key's are all taken; the candidates add their own bits later
      const uint64_t ma = __ballot((kv[u] & pmask) > pre);
      if (lane == 0 && c + u < V) {
        sm.bal[0][(c + u) * NW + w] = ma;
        sm.bal[1][(c + u) * NW + w] = 0ull;
      }
    }
  }
  __syncthreads();
  const uint32_t nc = min(sm.ncand, (uint32_t)TS_CCAP);
  uint32_t T, krem;
  if (nc <= (uint32_t)TS_WCAP) {
    if (w == 0) {
      // the bin_rank-th largest of the nc keys, bit by bit below the bin's 11 bits
      uint32_t kk[TS_WCAP / 64];
#pragma unroll
      for (int u = 0; u < TS_WCAP / 64; ++u) {
        const uint32_t j = 64u * u + lane;
        kk[u] = j < nc ? sm.cand[j] : 0u;
      }
      uint32_t t = pre;
      for (int b = low - 1; b >= 0; --b) {
        const uint32_t c = t | (1u << b);
        uint32_t cnt = 0;
#pragma unroll
        for (int u = 0; u < TS_WCAP / 64; ++u) cnt += (uint32_t)__popcll(__ballot(kk[u] >= c));
        if (cnt >= rank) t = c;
      }
      uint32_t gt = 0;
#pragma unroll
      for (int u = 0; u < TS_WCAP / 64; ++u) gt += (uint32_t)__popcll(__ballot(kk[u] > t));
      if (lane == 0) {
        sm.sh_digit = t;
        sm.sh_krem = rank - gt;
      }
    }
    __syncthreads();
    T = sm.sh_digit;
    krem = sm.sh_krem;
  } else {
    lds_select(sm.cand, (int)nc, rank, sm.hist, &sm.sh_digit, &sm.sh_krem, T, krem, 3, low == 21 ? 1 : 2, pre);
  }

  // the candidates above and equal to T set their bits (a key with a higher prefix has its bit
  // already); then the per-(v, w) counts, and one scan of them
  for (uint32_t j = tid; j < nc; j += TS_THREADS) {
    const uint32_t kv = sm.cand[j];
    if (kv >= T) {
      const int32_t p = sm.cpos[j];
      atomicOr((unsigned long long*)&sm.bal[kv > T ? 0 : 1][(p / TS_THREADS) * NW + (p % TS_THREADS) / 64],
               1ull << (p % 64));
    }
  }
  __syncthreads();
  for (int e = tid; e < V * NW; e += TS_THREADS) {
    sm.tab[e] = (uint32_t)__popcll(sm.bal[0][e]);
    sm.tab2[e] = (uint32_t)__popcll(sm.bal[1][e]);
  }
  __syncthreads();
  table_exclusive_scan2(sm.tab, sm.tab2, V * NW, sm.wt);
  // output position of entry (v, w, lane) if it is taken, else -1
  auto place = [&](int v) -> int32_t {
    const int j = v * NW + w;
    const uint64_t ma = sm.bal[0][j], me = sm.bal[1][j];
    const bool above = (ma >> lane) & 1u, equal = (me >> lane) & 1u;
    const uint32_t ab = sm.tab[j] + lanes_below(ma), eb = sm.tab2[j] + lanes_below(me);
    const bool take = above || (equal && eb < krem);
    return take ? (int32_t)(ab + min(eb, krem)) : -1;
  };
  if (k <= TS_OCAP) {
    // 8 values at a time, so that their LDS reads are in flight together
    for (int v0 = 0; v0 < V; v0 += 8) {
      int32_t pos[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) pos[u] = v0 + u < V ? place(v0 + u) : -1;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (pos[u] >= 0 && pos[u] < k) sm.osrc[pos[u]] = tid + TS_THREADS * (v0 + u);
    }
    __syncthreads();
    constexpr int PO = TS_OCAP / TS_THREADS;
    int32_t iv[PO];
    float yv[PO];
#pragma unroll
    for (int u = 0; u < PO; ++u) {
      const int p = tid + TS_THREADS * u;
      const int32_t src = p < k ? min(max(sm.osrc[p], 0), M - 1) : 0;
      iv[u] = p < k ? idx[src] : 0;
      yv[u] = (outs && p < k) ? ys[src] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < PO; ++u) {
      const int p = tid + TS_THREADS * u;
      if (p < k) {
        out[p] = iv[u];
        if (outs) outs[p] = yv[u];
      }
    }
    return true;
  }
  // larger k: each thread stores its own taken entries, 8 values at a time
  for (int c = 0; c < V; c += 8) {
    int32_t pos[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) pos[u] = c + u < V ? place(c + u) : -1;
    int32_t iv[8];
    float yv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = min(tid + TS_THREADS * (c + u), M - 1);
      iv[u] = pos[u] >= 0 ? idx[i] : 0;
      yv[u] = (outs && pos[u] >= 0) ? ys[i] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (pos[u] >= 0 && pos[u] < k) {
        out[pos[u]] = iv[u];
        if (outs) outs[pos[u]] = yv[u];
      }
  }
  return true;
}

// Radix select that re-reads the scores from memory on every pass (lists of
// any length): four 8-bit passes, then an ordered output pass in chunks of
// 1024 entries.
__device__ __forceinline__ void select_streaming(const float* __restrict__ ys, const int32_t* __restrict__ idx,
                                                 int32_t M, int32_t k, int32_t* out, float* outs) {
  const int tid = threadIdx.x;
  __shared__ uint32_t hist8[256];
  __shared__ uint32_t sd, sk;
  __shared__ uint32_t wt[TS_THREADS / 64];
  uint32_t prefix = 0, pmask = 0, krem = (uint32_t)k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) hist8[tid] = 0;
    __syncthreads();
    for (int32_t i = tid; i < M; i += TS_THREADS) {
      const uint32_t u = order_key(ys[i]);
      if ((u & pmask) == prefix) atomicAdd(&hist8[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // lane j owns bins 4j..4j+3; suffix sums from the top bin down
      uint32_t s4[4], own = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) { s4[i] = hist8[4 * tid + i]; own += s4[i]; }
      uint32_t suf = own;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_down(suf, o);
        if (tid + o < 64) suf += y;
      }
      const uint32_t above = suf - own;
      if (above < krem && krem <= suf) {
        uint32_t cum = above;
        for (int i = 3; i >= 0; --i) {
          if (cum + s4[i] >= krem) {
            sd = 4 * tid + i;
            sk = krem - cum;
            break;
          }
          cum += s4[i];
        }
      }
    }
    __syncthreads();
    prefix |= sd << shift;
    pmask |= 255u << shift;
    krem = sk;
    __syncthreads();
  }
  const uint32_t T = prefix;
  int64_t run_out = 0, run_eq = 0;
  for (int32_t base_i = 0; base_i < M; base_i += TS_THREADS) {
    const int32_t i = base_i + tid;
    const bool in = i < M;
    const float y = in ? ys[i] : 0.0f;
    const uint32_t u = in ? order_key(y) : 0u;
    const bool gt = in && u > T;
    const bool eq = in && u == T;
    uint32_t tot_eq, tot_take;
    const int64_t eq_before = run_eq + block_prefix_small<1>(eq ? 1u : 0u, wt, tot_eq);
    const bool take = gt || (eq && eq_before < (int64_t)krem);
    const int64_t pos = run_out + block_prefix_small<1>(take ? 1u : 0u, wt, tot_take);
    if (take) {
      out[pos] = idx[i];
      if (outs) outs[pos] = y;
    }
    run_out += tot_take;
    run_eq += tot_eq;
  }
}

// Radix select over n <= TS_FCAP keys held in LDS: T = the key of the rank-th
// largest, and krem = how many of the keys equal to T are among the first
// `rank` (the rest of those equal to T rank after them). Thread t handles
// keys t, t + TS_THREADS, ...
static constexpr int TS_FCAP = 4096;     // candidates kept after the filter

// With first_pass = 1 the top 11 bits are already known (first_pass = 2: the top
// 22 bits): prefix holds them and only keys with those bits take part (rank
// counts among them).
__device__ __forceinline__ void lds_select(const uint32_t* keys, int n, uint32_t rank, uint32_t* hist,
                                           uint32_t* sh_digit, uint32_t* sh_krem, uint32_t& T, uint32_t& krem,
                                           int passes, int first_pass, uint32_t prefix) {
  const int tid = threadIdx.x;
  uint32_t pmask = first_pass == 0 ? 0u : (first_pass == 1 ? 0xFFE00000u : 0xFFFFFC00u);
  krem = rank;
  for (int pass = first_pass; pass < passes; ++pass) {
    const int sh = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nb = pass == 2 ? 1024 : 2048;
    for (int i = tid; i < 2048; i += TS_THREADS) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += TS_THREADS) {
      const uint32_t kv = keys[i];
      if ((kv & pmask) == prefix) atomicAdd(&hist[(kv >> sh) & (nb - 1)], 1u);
    }
    __syncthreads();
    find_digit(hist, nb, krem, sh_digit, sh_krem);
    prefix |= *sh_digit << sh;
    pmask |= (uint32_t)(nb - 1) << sh;
    krem = *sh_krem;
    __syncthreads();
  }
  T = prefix;
}

// Select through the k-th key's histogram bin. The scoring kernel counted the
// list's keys by their top 11 bits, so the bin d holding the k-th largest key
// and the number of keys in higher bins are known exactly. One pass keeps the
// entries with key >= t = d << 21 (the bin and everything above it), in list
// order (each thread owns a contiguous run of the list, so one block scan
// places them); there are between k and k + hist[d] of them. The exact select
// then ranks only the keys of bin d, on their lower 21 bits. Returns false,
// having written nothing, when the kept entries do not fit in TS_FCAP; the
// caller then runs a full select.
#define LSA_GLOBAL __attribute__((address_space(1)))
__device__ __forceinline__ bool select_filtered(const float* __restrict__ ys_, const int32_t* __restrict__ idx_,
                                                int32_t M, int32_t k, int32_t* out_, float* outs_,
                                                const uint32_t* __restrict__ hist_) {
  // Global-memory pointers: the accesses below are global loads and stores, never generic
  // (flat) ones, which would wait for every outstanding memory and LDS operation.
  const LSA_GLOBAL float* ys = (const LSA_GLOBAL float*)ys_;
  const LSA_GLOBAL int32_t* idx = (const LSA_GLOBAL int32_t*)idx_;
  LSA_GLOBAL int32_t* out = (LSA_GLOBAL int32_t*)out_;
  LSA_GLOBAL float* outs = (LSA_GLOBAL float*)outs_;
  const int tid = threadIdx.x;
  __shared__ uint32_t fkey[TS_FCAP];    // the kept keys
  __shared__ int32_t fpos[TS_FCAP];     // list positions of the kept keys
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t sh_digit, sh_krem;
  __shared__ uint32_t wt[TS_THREADS / 64];

  // 1. the bin of the k-th largest key, from the scoring kernel's histogram
  // of the top 11 key bits: t = the bin's smallest key. Exactly `above`
  // entries lie in higher bins and hist[d] in the bin, so the kept count is
  // known before the pass.
  const LSA_GLOBAL uint32_t* hg = (const LSA_GLOBAL uint32_t*)hist_;
  for (int j = tid; j < 2048; j += TS_THREADS) hist[j] = hg[j];
  __syncthreads();
  find_digit(hist, 2048, (uint32_t)k, &sh_digit, &sh_krem);
  const uint32_t d = sh_digit;
  const uint32_t bin_krem = sh_krem;  // rank of the k-th key among the keys of its bin
  const uint32_t kept = (uint32_t)k - bin_krem + hist[d];
  __syncthreads();
  if (kept > (uint32_t)TS_FCAP) return false;  // uniform
  const uint32_t t = d << 21;

  // 2. keep the entries with key >= t, in list order. Rounds of TS_THREADS x 8
  // entries; thread j owns entries 8j .. 8j+7 of a round, so the loads of a
  // wave cover 2 KiB, and one block prefix per round places the kept entries.
  // The loads of up to FR rounds are issued together before any is used, so
  // a list of up to FR x 8192 entries costs one memory round trip.
  constexpr int FR = 2;
  int32_t c = 0;  // kept so far (the same in every thread)
  for (int32_t cbase = 0; cbase < M; cbase += FR * TS_THREADS * 8) {
    // raw scores first (clamped indices, no branch), keys only when used, so
    // all the loads are in flight together
    float yv[FR][8];
#pragma unroll
    for (int r = 0; r < FR; ++r) {
      const int32_t i0 = cbase + r * TS_THREADS * 8 + 8 * tid;
#pragma unroll
      for (int u = 0; u < 8; ++u) yv[r][u] = ys[min(i0 + u, M - 1)];
    }
#pragma unroll
    for (int r = 0; r < FR; ++r) {
      const int32_t rbase = cbase + r * TS_THREADS * 8;
      if (rbase < M) {  // uniform
        const int32_t i0 = rbase + 8 * tid;
        uint32_t kv[8], keep = 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          kv[u] = order_key(yv[r][u]);
          keep |= (i0 + u < M && kv[u] >= t) ? 1u << u : 0u;
        }
        uint32_t tot;
        const uint32_t off = block_prefix_small<4>((uint32_t)__builtin_popcount(keep), wt, tot);
        if (c + (int32_t)tot > TS_FCAP) return false;     // uniform: tot is the block total
        int32_t o = c + (int32_t)off;
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (keep & (1u << u)) {
            fkey[o] = kv[u];
            fpos[o] = i0 + u;
            ++o;
          }
        c += (int32_t)tot;
      }
    }
  }
  if (c < k) return false;
  __syncthreads();

  // 3. exact select among the kept entries of the k-th bin (the top 11 bits are d)
  uint32_t T, krem;
  lds_select(fkey, c, bin_krem, hist, &sh_digit, &sh_krem, T, krem, 3, 1, t);

  // 4. output: keys above T, and the first krem keys equal to T, in list order
  const int32_t q = (c + TS_THREADS - 1) / TS_THREADS;
  const int32_t j0 = min(c, tid * q), j1 = min(c, j0 + q);
  int32_t neq = 0;
  for (int32_t j = j0; j < j1; ++j) neq += fkey[j] == T ? 1 : 0;
  uint32_t tot_eq;
  int64_t eq_before = block_prefix_small<3>((uint32_t)neq, wt, tot_eq);  // neq <= 4
  int32_t ntake = 0;
  {
    int64_t e = eq_before;
    for (int32_t j = j0; j < j1; ++j) {
      const uint32_t kv = fkey[j];
      const bool take = kv > T || (kv == T && e < (int64_t)krem);
      if (kv == T) ++e;
      ntake += take ? 1 : 0;
    }
  }
  uint32_t tot_take;
  int32_t pos = (int32_t)block_prefix_small<3>((uint32_t)ntake, wt, tot_take);   // ntake <= 4
  // this thread's (at most 4) outputs: positions, then all the loads, then the stores
  // (slot s of src takes the s-th taken entry; every index is a constant, so src stays in registers)
  int32_t src[4] = {0, 0, 0, 0};
  int nt = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int32_t j = j0 + u;
    if (j < j1) {
      const uint32_t kv = fkey[j];
      const bool take = kv > T || (kv == T && eq_before < (int64_t)krem);
      if (kv == T) ++eq_before;
      const int32_t fp = fpos[j];
#pragma unroll
      for (int s = 0; s < 4; ++s) src[s] = (take && nt == s) ? fp : src[s];
      nt += take ? 1 : 0;
    }
  }
  int32_t iv[4];
  float yo[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    iv[u] = idx[src[u]];
    yo[u] = ys[src[u]];
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (u < nt && pos + u < k) {  // exactly k are taken; the bound only guards a mismatched workspace
      out[pos + u] = iv[u];
      if (outs) outs[pos + u] = yo[u];
    }
  return true;
}

__global__ __launch_bounds__(TS_THREADS) void topk_select_kernel(const TopkSelectArgs a) {
  __shared__ RegSelectSmem rsm;
  const int b = blockIdx.x, l = blockIdx.y, tid = threadIdx.x;
  const int64_t base = a.key_off[b];
  const int32_t M = a.count[b];
  const int32_t k = a.k;
  const float* ys = a.ys + (int64_t)l * a.rows_total + base;
  const int32_t* idx = a.idx + base;
  int32_t* out = a.out_idx[l] + (int64_t)b * k;
  float* outs = a.out_score[l] ? a.out_score[l] + (int64_t)b * k : nullptr;
  const uint32_t* hb = a.hist ? a.hist + ((int64_t)l * a.B + b) * TOPK_BINS : nullptr;
  if (M <= k) {
    for (int32_t i = tid; i < k; i += TS_THREADS) {
      out[i] = i < M ? idx[i] : -1;
      if (outs) outs[i] = i < M ? ys[i] : -INFINITY;
    }
  } else if (M <= TS_THREADS * TS_VMAX) {
    // without the scorer's histogram the register select counts the bins itself (radix passes)
    if (M <= TS_THREADS * 8) select_in_registers<8>(ys, idx, M, k, out, outs, hb, rsm);
    else if (M <= TS_THREADS * 16) select_in_registers<16>(ys, idx, M, k, out, outs, hb, rsm);
    else select_in_registers<TS_VMAX>(ys, idx, M, k, out, outs, hb, rsm);
  } else if (M <= TS_THREADS * TS_RMAX && select_reload(ys, idx, M, k, out, outs, hb, rsm)) {
    // done with the scores read again from memory
  } else if (hb && (int64_t)k * 2 <= TS_FCAP && select_filtered(ys, idx, M, k, out, outs, hb)) {
    // done through the histogram's bin of the k-th key
  } else {
    select_streaming(ys, idx, M, k, out, outs);
  }
  if (tid == 0) a.out_count[l * gridDim.x + b] = M < k ? M : k;
}

hipError_t launch_topk_select(const TopkSelectArgs& a, int L, hipStream_t st) {
  hipLaunchKernelGGL(topk_select_kernel, dim3(a.B, L), dim3(TS_THREADS), 0, st, a);
  return hipGetLastError();
}

}  // namespace lsa
