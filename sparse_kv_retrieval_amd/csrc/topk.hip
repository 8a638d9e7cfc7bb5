// Top-k inside the loaded subset: the second level of the two-level selection
// ([BLOG] §3.2 of the FlashMemory-DeepSeek-V4 write-up: the native Lightning
// Indexer picks the final top-k core entries inside C^MemComp).
//
// One block per (sequence, layer). The scores y are in the workspace, in
// subset order, which is ascending entry order. A radix select over
// order-preserving uint32 keys finds T, the key of the k-th largest score, and
// how many entries equal to T must be kept. The output keeps every entry above
// T plus the lowest-index entries equal to it, in list order, which matches
// the (-y, s) order and keeps the output ascending.
#include "kernels.hpp"

namespace lsa {

static constexpr int TS_THREADS = 1024;
static constexpr int TS_VMAX = 80;  // values per thread held in registers (lists up to 81,920)

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

// Exclusive scan, in place, of an LDS table of n <= 2 * TS_THREADS counts.
__device__ __forceinline__ void table_exclusive_scan(uint32_t* tab, int n) {
  const int tid = threadIdx.x;
  const int j0 = 2 * tid;
  const uint32_t a0 = j0 < n ? tab[j0] : 0u, a1 = j0 + 1 < n ? tab[j0 + 1] : 0u;
  __shared__ uint32_t wt[TS_THREADS / 64];
  uint32_t tot;
  const uint32_t ex = block_prefix_small<8>(a0 + a1, wt, tot);  // a0, a1 <= 64
  if (j0 < n) tab[j0] = ex;
  if (j0 + 1 < n) tab[j0 + 1] = ex + a0;
  __syncthreads();
}

// Radix select over a list held in registers.
//
// Thread t = 64 w + lane holds the list entries i = t + 1024 v (v < V), so
// every load is coalesced. Three histogram passes over bits 31..21, 20..10
// and 9..0 of the keys touch only registers and a 2048-bin LDS histogram, and
// find T, the key of the k-th largest score. The list order is (v, w, lane).
// An entry's rank among the entries before it is therefore a count of lanes
// below it in its wave (ballot + mbcnt) plus an exclusive scan of the
// per-(v, w) counts held in a small LDS table. One such scan ranks the entries
// equal to T, which settles ties toward the lower index. A second one places
// each kept entry at its ascending output position.
__device__ __forceinline__ void select_in_registers(const float* __restrict__ ys, const int32_t* __restrict__ idx,
                                                    int32_t M, int32_t k, int32_t* out, float* outs) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  constexpr int NW = TS_THREADS / 64;
  const int V = (M + TS_THREADS - 1) / TS_THREADS;
  // Key 0 pads the tail. It sorts below every real key (the smallest real key,
  // -inf, maps to 0x007FFFFF), so padding never reaches the selected bins or
  // the output, and the passes need no bounds test.
  // Loads go in chunks of 8 with clamped addresses, so each chunk is one round trip.
  uint32_t key[TS_VMAX];
#pragma unroll
  for (int c = 0; c < TS_VMAX; c += 8) {
    if (c < V) {
      float y[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) y[u] = ys[min(tid + TS_THREADS * (c + u), M - 1)];
#pragma unroll
      for (int u = 0; u < 8; ++u) key[c + u] = (c + u < V && tid + TS_THREADS * (c + u) < M) ? order_key(y[u]) : 0u;
    }
  }

  __shared__ uint32_t hist[2048];
  __shared__ uint32_t tab[TS_VMAX * NW], tab2[TS_VMAX * NW];
  __shared__ uint32_t sh_digit, sh_krem;
  uint32_t prefix = 0, pmask = 0, krem = (uint32_t)k;
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int sh = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nb = pass == 2 ? 1024 : 2048;
    for (int i = tid; i < 2048; i += TS_THREADS) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int v = 0; v < TS_VMAX; ++v)
      if (v < V && (key[v] & pmask) == prefix) atomicAdd(&hist[(key[v] >> sh) & (nb - 1)], 1u);
    __syncthreads();
    find_digit(hist, nb, krem, &sh_digit, &sh_krem);
    prefix |= sh_digit << sh;
    pmask |= (uint32_t)(nb - 1) << sh;
    krem = sh_krem;
    __syncthreads();
  }
  const uint32_t T = prefix;

  // Ballots are recomputed in each loop rather than kept, so registers hold only the keys.
  // tab holds per-(v, w) counts of entries equal to T, then their exclusive scan;
  // tab2 the same for kept entries.
#pragma unroll
  for (int v = 0; v < TS_VMAX; ++v)
    if (v < V) {
      const uint64_t m = __ballot(key[v] == T);
      if (lane == 0) tab[v * NW + w] = (uint32_t)__popcll(m);
    }
  __syncthreads();
  table_exclusive_scan(tab, V * NW);
#pragma unroll
  for (int v = 0; v < TS_VMAX; ++v)
    if (v < V) {
      const uint64_t meq = __ballot(key[v] == T);
      const bool take = key[v] > T || (key[v] == T && tab[v * NW + w] + lanes_below(meq) < krem);
      const uint64_t mt = __ballot(take);
      if (lane == 0) tab2[v * NW + w] = (uint32_t)__popcll(mt);
    }
  __syncthreads();
  table_exclusive_scan(tab2, V * NW);
  // output in chunks of 8: positions first, then all the loads, then all the stores
#pragma unroll
  for (int c = 0; c < TS_VMAX; c += 8) {
    if (c < V) {
      int32_t pos[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int v = c + u;
        pos[u] = -1;
        if (v < V) {
          const uint64_t meq = __ballot(key[v] == T);
          const bool take = key[v] > T || (key[v] == T && tab[v * NW + w] + lanes_below(meq) < krem);
          const uint64_t mt = __ballot(take);
          if (take) pos[u] = (int32_t)(tab2[v * NW + w] + lanes_below(mt));
        }
      }
      int32_t iv[8];
      float yv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = min(tid + TS_THREADS * (c + u), M - 1);
        iv[u] = pos[u] >= 0 ? idx[i] : 0;
        yv[u] = (outs && pos[u] >= 0) ? ys[i] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (pos[u] >= 0) {
          out[pos[u]] = iv[u];
          if (outs) outs[pos[u]] = yv[u];
        }
      }
    }
  }
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
static constexpr int TS_SAMPLE = 4096;   // sampled scores for the threshold estimate

__device__ __forceinline__ void lds_select(const uint32_t* keys, int n, uint32_t rank, uint32_t* hist,
                                           uint32_t* sh_digit, uint32_t* sh_krem, uint32_t& T, uint32_t& krem,
                                           int passes = 3) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, pmask = 0;
  krem = rank;
  for (int pass = 0; pass < passes; ++pass) {
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

// Select through a threshold estimated from a sample. TS_SAMPLE scores at
// evenly spaced list positions give t, the sample key of rank
// r = ceil(k S / M) * 5/4 + 32: about 1.25 k + 32 M/S entries of the list are
// expected at or above it, so at least k with a wide margin. One pass keeps
// the entries with key >= t, in list order (each thread owns a contiguous run
// of the list, so one block scan places them), as long as they number between
// k and TS_FCAP. The exact select then runs on those. Every entry of the top k
// has key >= the k-th key >= t whenever at least k keys are >= t, so the
// result is the exact top-k. Returns false, having written nothing, when the
// kept count falls outside [k, TS_FCAP]; the caller then runs a full select.
#define LSA_GLOBAL __attribute__((address_space(1)))
__device__ __attribute__((noinline)) bool select_filtered(const float* __restrict__ ys_, const int32_t* __restrict__ idx_,
                                                int32_t M, int32_t k, int32_t* out_, float* outs_) {
  // This function is not inlined, so its pointer arguments lose the knowledge
  // that they point to global memory; generic (flat) accesses would make every
  // load wait for all outstanding memory and LDS operations. Restore it.
  const LSA_GLOBAL float* ys = (const LSA_GLOBAL float*)ys_;
  const LSA_GLOBAL int32_t* idx = (const LSA_GLOBAL int32_t*)idx_;
  LSA_GLOBAL int32_t* out = (LSA_GLOBAL int32_t*)out_;
  LSA_GLOBAL float* outs = (LSA_GLOBAL float*)outs_;
  const int tid = threadIdx.x;
  __shared__ uint32_t fkey[TS_FCAP];    // sampled keys, then the kept keys
  __shared__ int32_t fpos[TS_FCAP];     // list positions of the kept keys
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t sh_digit, sh_krem;
  __shared__ uint32_t wt[TS_THREADS / 64];

  // 1. threshold estimate from the sample. Two radix passes fix the top 22
  // bits of the rank-r sample key; t (those bits, the rest zero) is at most
  // that key, so at least as many entries pass as with the exact key.
  for (int j = tid; j < TS_SAMPLE; j += TS_THREADS)
    fkey[j] = order_key(ys[(int32_t)((int64_t)j * M / TS_SAMPLE)]);
  __syncthreads();
  const uint32_t est = (uint32_t)(((int64_t)k * TS_SAMPLE + M - 1) / M);
  const uint32_t r = min((uint32_t)TS_SAMPLE, est + est / 4 + 32);
  uint32_t t, tk;
  lds_select(fkey, TS_SAMPLE, r, hist, &sh_digit, &sh_krem, t, tk, 2);

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

  // 3. exact select among the kept entries
  uint32_t T, krem;
  lds_select(fkey, c, (uint32_t)k, hist, &sh_digit, &sh_krem, T, krem);

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
  int32_t src[4];
  int nt = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int32_t j = j0 + u;
    src[u] = 0;
    if (j < j1) {
      const uint32_t kv = fkey[j];
      const bool take = kv > T || (kv == T && eq_before < (int64_t)krem);
      if (kv == T) ++eq_before;
      if (take) src[nt++] = fpos[j];
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
    if (u < nt) {
      out[pos + u] = iv[u];
      if (outs) outs[pos + u] = yo[u];
    }
  return true;
}

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
  } else if (M >= 2 * TS_SAMPLE && (int64_t)k * 4 <= TS_FCAP * 3 && select_filtered(ys, idx, M, k, out, outs)) {
    // done through the sample threshold
  } else if (M <= TS_THREADS * TS_VMAX) {
    select_in_registers(ys, idx, M, k, out, outs);
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
