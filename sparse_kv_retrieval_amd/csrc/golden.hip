// Golden-label mining: the training targets of the memory indexer.
//
// hyper.ai digest of FlashMemory-DeepSeek-V4, "数据集" (Dataset), and the
// marsggbo write-up, §4.1 "Golden Label 怎么造": for every token of the
// lookahead window and every CSA layer, the raw indexer logits over the
// token's preceding compressed entries are normalised by a softmax and cut by
// a top-p nucleus (p = 0.6). An entry is golden for the token when at least
// theta = 3 layers keep it; the window's label set is the union over its
// tokens. The gist.science summary, §2.2, states the same three steps.
//
// Nucleus: entries ordered by descending logit (equal logits by ascending
// entry index); an entry is kept while the probability mass of the entries
// before it is below p. Equivalently there is a key T (the order-preserving
// uint32 image of the crossing entry's logit) and an index cut such that an
// entry is kept iff key > T, or key == T and index <= cut.
//
// Kernel 1 (one 1024-thread block per (token, layer) row):
//   pass A  streams the row from HBM once: a running block maximum M and a
//           4096-bin histogram of the masses exp(y - M) over the top 12 key
//           bits (fp64 LDS atomics, rescaled whenever M grows);
//   scan    finds the crossing bin b1 of the cumulative mass (descending keys)
//           at p * Z, Z the histogram total;
//   pass B  streams the row again: entries above b1 are written as kept into
//           the row's bit mask, entries in b1 go to an LDS candidate list;
//   levels  two 10-bit levels over the candidates find T exactly, the count of
//           entries equal to T that are kept follows from their common mass,
//           and if that is not all of them a 3 x 10-bit count select over
//           their indices finds the cut;
//   fix-up  kept candidates are OR-ed into the mask words.
// If the crossing bin holds more candidates than the LDS list, every level
// reads the row instead of the list and a final pass rewrites the mask.
//
// Kernel 2 (vote and union): per (token, mask word), a bit-sliced count of the
// layers' mask bits, compared with theta, and OR-ed over the window's tokens.
#include "kernels.hpp"

namespace lsa {

namespace {

constexpr int GT = 1024;          // threads per nucleus block
constexpr int GW = GT / 64;       // waves per nucleus block
constexpr int GLL = 16;           // dword loads per lane per wave chunk
constexpr int GWC = 64 * GLL;     // entries per wave chunk: 16 mask words
constexpr int GBC = GWC * GW;     // entries per block chunk
constexpr int NB1 = 4096;         // level-1 bins: key bits 31..20
constexpr int NBL = 1024;         // later levels: 10 bits, one bin per thread
constexpr int GCAP = 4096;        // candidates held in LDS
constexpr uint32_t NONE = 0xFFFFFFFFu;
constexpr float LOG2E = 1.4426950408889634f;

struct GoldenSmem {
  double bins[NB1];    // level-1 masses; levels 2-3 use the first NBL
  uint32_t cnt[NBL];   // per-digit counts of levels 2-3 and of the index select
  uint32_t ckey[GCAP];
  uint32_t cidx[GCAP];
  double wsum[GW];
  uint32_t usum[GW];
  float wmax[2][GW];
  double res_A;
  uint32_t res_digit, res_cnt, ncand, kept;
  int32_t last;
};

__device__ __forceinline__ float key_value(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// Unnormalised probability of a logit relative to the row maximum M.
__device__ __forceinline__ float rel_mass(float y, float M) { return __builtin_amdgcn_exp2f((y - M) * LOG2E); }

__device__ __forceinline__ uint32_t below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ void lds_add(double* p, double v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_inc(uint32_t* p) {
  __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Inclusive and exclusive block-wide prefix sums of one double per thread, in
// thread order, and the block total. excl of thread t + 1 equals incl of
// thread t bit for bit, so the running sums are exactly monotone.
__device__ __forceinline__ void block_scan_f64(double v, GoldenSmem& sm, double& excl, double& incl, double& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  double x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  const double prev = __shfl_up(x, 1);
  if (lane == 63) sm.wsum[w] = x;
  __syncthreads();
  double off = 0.0, tot = 0.0;
  for (int i = 0; i < GW; ++i) {
    if (i == w) off = tot;
    tot += sm.wsum[i];
  }
  __syncthreads();
  incl = off + x;
  excl = lane == 0 ? off : off + prev;
  total = tot;
}

// The same for uint32 counts (exact).
__device__ __forceinline__ void block_scan_u32(uint32_t v, GoldenSmem& sm, uint32_t& excl, uint32_t& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sm.usum[w] = x;
  __syncthreads();
  uint32_t off = 0, tot = 0;
  for (int i = 0; i < GW; ++i) {
    off += i < w ? sm.usum[i] : 0u;
    tot += sm.usum[i];
  }
  __syncthreads();
  excl = off + x - v;
  total = tot;
}

// Where the level's items come from: the LDS candidate list, or the whole row.
struct FromList {
  const GoldenSmem* sm;
  uint32_t n;
  template <class F>
  __device__ __forceinline__ void each(F&& f) const {
    for (uint32_t j = threadIdx.x; j < n; j += GT) f(sm->ckey[j], sm->cidx[j]);
  }
};
struct FromRow {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t n;
  template <class F>
  __device__ __forceinline__ void each(F&& f) const {
    for (uint32_t e0 = 0; e0 < n; e0 += 4 * GT) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = __uint_as_float(buf_load4(rs, (e0 + u * GT + threadIdx.x) * 4u));
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t e = e0 + u * GT + threadIdx.x;
        if (e < n) f(order_key(v[u]), e);
      }
    }
  }
};

// One 10-bit mass level: among items whose key >> (sh + 10) equals pre, the
// digit (key >> sh) & 1023 where the cumulative mass, taken in descending key
// order on top of A (the mass of every key above the prefix), reaches target.
// Returns the digit, the mass above it and its count. When rounding leaves the
// sum short of the target, the lowest non-empty digit is taken.
template <class Src>
__device__ void mass_level(GoldenSmem& sm, const Src& src, uint32_t pre, int sh, float M, double target, double& A,
                           uint32_t& digit, uint32_t& count) {
  const int t = threadIdx.x;
  __syncthreads();  // earlier readers of bins / cnt are done
  sm.bins[t] = 0.0;
  sm.cnt[t] = 0;
  if (t == 0) {
    sm.res_digit = NONE;
    sm.last = -1;
  }
  __syncthreads();
  src.each([&](uint32_t key, uint32_t) {
    if ((key >> (sh + 10)) == pre) {
      const uint32_t d = (key >> sh) & (NBL - 1);
      lds_add(&sm.bins[d], (double)rel_mass(key_value(key), M));
      lds_inc(&sm.cnt[d]);
    }
  });
  __syncthreads();
  const uint32_t d = NBL - 1 - t;  // thread order = descending digit
  const double m = sm.bins[d];
  const uint32_t c = sm.cnt[d];
  double ex, in, tot;
  block_scan_f64(m, sm, ex, in, tot);
  if (A + ex < target && A + in >= target) {
    sm.res_digit = d;
    sm.res_A = A + ex;
    sm.res_cnt = c;
  }
  if (c > 0) atomicMax(&sm.last, t);
  __syncthreads();
  if (sm.res_digit != NONE) {
    digit = sm.res_digit;
    A = sm.res_A;
    count = sm.res_cnt;
  } else if (sm.last >= 0) {
    const uint32_t dl = NBL - 1 - (uint32_t)sm.last;
    digit = dl;
    A = A + (tot - sm.bins[dl]);
    count = sm.cnt[dl];
  } else {  // no item under the prefix (not reached: the prefix always holds the crossing entry)
    digit = 0;
    count = 0;
  }
}

// The rank-th smallest index (rank >= 1) among items with key == T, by three
// 10-bit count levels over the index bits 29..0.
template <class Src>
__device__ uint32_t index_select(GoldenSmem& sm, const Src& src, uint32_t T, uint32_t rank) {
  const int t = threadIdx.x;
  uint32_t pre = 0;
  for (int sh = 20; sh >= 0; sh -= 10) {
    __syncthreads();
    sm.cnt[t] = 0;
    if (t == 0) sm.res_digit = NONE;
    __syncthreads();
    src.each([&](uint32_t key, uint32_t idx) {
      if (key == T && (idx >> (sh + 10)) == pre) lds_inc(&sm.cnt[(idx >> sh) & (NBL - 1)]);
    });
    __syncthreads();
    const uint32_t c = sm.cnt[t];
    uint32_t ex, tot;
    block_scan_u32(c, sm, ex, tot);
    if (ex < rank && ex + c >= rank) {
      sm.res_digit = t;
      sm.res_cnt = ex;
    }
    __syncthreads();
    pre = (pre << 10) | sm.res_digit;
    rank -= sm.res_cnt;
  }
  return pre;
}

// The loads of one wave chunk: lane j of load k reads entry base + 64k + j, so
// the ballot of load k is mask word base / 64 + k. The offset is one VGPR, which
// the buffer's range check covers (entries at or beyond n read as 0 without a
// memory access); the 64k part goes in the instruction's immediate offset.
__device__ __forceinline__ void load_chunk(const __amdgpu_buffer_rsrc_t rs, uint32_t voff, float (&v)[GLL]) {
  int vo = (int)voff;  // < 2^31; a signed add lets the constant fold into the immediate
  asm("" : "+v"(vo));  // one offset register per chunk, not one induction variable per load
#pragma unroll
  for (int k = 0; k < GLL; ++k)
    v[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, vo + 256 * k, 0, 0));
}

// Runs body(v, base) over the wave's chunks of the row (chunk it starts at
// entry (it * GW + wv) * GWC) with the next chunk's loads in flight while the
// current one is processed. Two named buffers and unconditional loads (past
// the row they read zeros) keep in-flight loads out of register copies, which
// would make the compiler wait for them.
template <class F>
__device__ __forceinline__ void stream_row(const __amdgpu_buffer_rsrc_t rs, uint32_t wv, uint32_t lane, uint32_t nit,
                                           F&& body) {
  float va[GLL], vb[GLL];
  load_chunk(rs, (wv * GWC + lane) * 4u, va);
  for (uint32_t it = 0;; it += 2) {
    load_chunk(rs, (((it + 1) * GW + wv) * GWC + lane) * 4u, vb);
    body(va, (it * GW + wv) * GWC);
    if (it + 1 >= nit) break;
    load_chunk(rs, (((it + 2) * GW + wv) * GWC + lane) * 4u, va);
    body(vb, ((it + 1) * GW + wv) * GWC);
    if (it + 2 >= nit) break;
  }
}

__global__ __launch_bounds__(GT) __attribute__((amdgpu_waves_per_eu(8, 8)))
void nucleus_kernel(const GoldenArgs a) {
  __shared__ GoldenSmem sm;
  const int t = threadIdx.x;
  const uint32_t wv = uni((int32_t)(t >> 6));  // wave-uniform
  const uint32_t lane = t & 63;
  const int row = blockIdx.x;
  const int tok = row / a.L;
  const int32_t nv = a.n_valid[tok];
  const uint32_t n = (uint32_t)min((int64_t)max(nv, 0), a.row_stride);
  const uint32_t nw = (n + 63) >> 6;
  const float* y = a.logits + (int64_t)row * a.row_stride;
  uint64_t* words = a.row_mask + (int64_t)row * a.W;
  const auto rs = buf_rsrc(y, n * 4u);

  if (row == 0)
    for (int64_t j = t; j < a.W; j += GT) a.golden[j] = 0;  // the vote kernel ORs into it
  for (uint32_t j = nw + t; j < (uint32_t)a.W; j += GT) words[j] = 0;
  if (n == 0) {
    if (a.nucleus_size && t == 0) a.nucleus_size[row] = 0;
    return;
  }

  // ---- pass A: maximum and level-1 mass histogram, one read of the row
#pragma unroll
  for (int j = 0; j < NB1 / GT; ++j) sm.bins[t * (NB1 / GT) + j] = 0.0;
  if (t == 0) {
    sm.ncand = 0;
    sm.kept = 0;
  }
  const uint32_t nit = (n + GBC - 1) / GBC;
  float M = -INFINITY;
  uint32_t par = 0;
  stream_row(rs, wv, lane, nit, [&](float (&v)[GLL], uint32_t base) {
    const bool full = base + GWC <= n;
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < GLL; ++k)
      if (full || base + 64u * k + lane < n) m = fmaxf(m, v[k]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if (lane == 0) sm.wmax[par][wv] = m;
    __syncthreads();
    float Mn = M;
#pragma unroll
    for (int j = 0; j < GW; ++j) Mn = fmaxf(Mn, sm.wmax[par][j]);
    par ^= 1;
    if (Mn > M) {  // the same decision in every thread
      if (M != -INFINITY) {
        const double f = (double)rel_mass(M, Mn);
#pragma unroll
        for (int j = 0; j < NB1 / GT; ++j) sm.bins[t * (NB1 / GT) + j] *= f;
      }
      M = Mn;
      __syncthreads();
    }
    if (full) {
#pragma unroll
      for (int k = 0; k < GLL; ++k) lds_add(&sm.bins[order_key(v[k]) >> 20], (double)rel_mass(v[k], M));
    } else {
#pragma unroll
      for (int k = 0; k < GLL; ++k)
        if (base + 64u * k + lane < n) lds_add(&sm.bins[order_key(v[k]) >> 20], (double)rel_mass(v[k], M));
    }
  });
  __syncthreads();

  // ---- level 1: crossing bin of the cumulative mass at p * Z
  double A, target;
  uint32_t b1;
  {
    double l[NB1 / GT], s = 0.0;  // this thread's bins, descending
#pragma unroll
    for (int j = 0; j < NB1 / GT; ++j) {
      s += sm.bins[NB1 - 1 - (NB1 / GT) * t - j];
      l[j] = s;
    }
    double ex, in, Z;
    block_scan_f64(s, sm, ex, in, Z);
    target = (double)a.p * Z;
    if (t == 0) sm.res_digit = NONE;
    __syncthreads();
    if (ex < target && in >= target) {
      // first of this thread's bins (descending) whose running sum reaches the
      // target; if rounding leaves it short, the last bin that holds mass
      int jj = -1, jm = 0;
      double above = ex, above_m = ex, prev = 0.0;
#pragma unroll
      for (int j = 0; j < NB1 / GT; ++j) {
        if (jj < 0 && ex + l[j] >= target) {
          jj = j;
          above = ex + prev;
        }
        if (l[j] > prev) {
          jm = j;
          above_m = ex + prev;
        }
        prev = l[j];
      }
      if (jj < 0) {
        jj = jm;
        above = above_m;
      }
      sm.res_digit = NB1 - 1 - (NB1 / GT) * t - jj;
      sm.res_A = above;
    }
    __syncthreads();
    b1 = sm.res_digit;
    A = sm.res_A;
  }

  // ---- pass B: mask words for decided entries, candidates of bin b1
  uint32_t kept = 0;
  stream_row(rs, wv, lane, nit, [&](float (&v)[GLL], uint32_t base) {
    uint64_t mine = 0;
#pragma unroll
    for (int k = 0; k < GLL; ++k) {
      const uint32_t e = base + 64u * k + lane;
      const uint32_t key = order_key(v[k]);
      const bool valid = e < n;
      const uint64_t kw = __ballot(valid && (key >> 20) > b1);
      const uint64_t cm = __ballot(valid && (key >> 20) == b1);
      kept += (uint32_t)__popcll(kw);
      mine = lane == (uint32_t)k ? kw : mine;
      if (cm) {
        uint32_t c0 = 0;
        if (lane == 0)
          c0 = __hip_atomic_fetch_add(&sm.ncand, (uint32_t)__popcll(cm), __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_WORKGROUP);
        c0 = __shfl(c0, 0);
        if (valid && (key >> 20) == b1) {
          const uint32_t pos = c0 + below(cm);
          if (pos < GCAP) {
            sm.ckey[pos] = key;
            sm.cidx[pos] = e;
          }
        }
      }
    }
    const uint32_t wi = (base >> 6) + lane;
    if (lane < GLL && wi < nw) words[wi] = mine;
  });
  if (lane == 0) __hip_atomic_fetch_add(&sm.kept, kept, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  // The mask stores are complete before any wave's fix-up atomic below. A
  // workgroup-scope release is enough (waves of one block share the L2 that
  // both go to); an agent-scope fence would write back the whole L2.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  const uint32_t nc = sm.ncand;

  // ---- levels 2 and 3, then the tie count and the index cut
  uint32_t T, ncut = 0x7FFFFFFFu;
  auto resolve = [&](const auto& src) {
    uint32_t d2, c2, d3, nT;
    mass_level(sm, src, b1, 10, M, target, A, d2, c2);
    mass_level(sm, src, (b1 << 10) | d2, 0, M, target, A, d3, nT);
    T = (b1 << 20) | (d2 << 10) | d3;
    const double wT = (double)rel_mass(key_value(T), M);
    const double q = (target - A) / wT;
    uint32_t c = nT;
    if (q < (double)nT) c = q <= 1.0 ? 1u : (uint32_t)ceil(q);
    if (c < nT) ncut = index_select(sm, src, T, c);
  };
  if (nc <= GCAP) {
    const FromList src{&sm, nc};
    resolve(src);
    uint32_t fixed = 0;
    for (uint32_t j = t; j < nc; j += GT) {
      const uint32_t key = sm.ckey[j], idx = sm.cidx[j];
      if (key > T || (key == T && idx <= ncut)) {
        __hip_atomic_fetch_or(&words[idx >> 6], (uint64_t)1 << (idx & 63), __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_WORKGROUP);
        ++fixed;
      }
    }
    if (fixed) __hip_atomic_fetch_add(&sm.kept, fixed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  } else {
    const FromRow src{rs, n};
    resolve(src);
    // rewrite every word; each word is stored by the same lane that stored it in pass B
    __syncthreads();
    if (t == 0) sm.kept = 0;
    __syncthreads();
    kept = 0;
    stream_row(rs, wv, lane, nit, [&](float (&v)[GLL], uint32_t base) {
      uint64_t mine = 0;
#pragma unroll
      for (int k = 0; k < GLL; ++k) {
        const uint32_t e = base + 64u * k + lane;
        const uint32_t key = order_key(v[k]);
        const uint64_t kw = __ballot(e < n && (key > T || (key == T && e <= ncut)));
        kept += (uint32_t)__popcll(kw);
        mine = lane == (uint32_t)k ? kw : mine;
      }
      const uint32_t wi = (base >> 6) + lane;
      if (lane < GLL && wi < nw) words[wi] = mine;
    });
    if (lane == 0) __hip_atomic_fetch_add(&sm.kept, kept, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  __syncthreads();
  if (a.nucleus_size && t == 0) a.nucleus_size[row] = (int32_t)sm.kept;
}

// Per (token, word): count the L layers' bits in 7 bit planes, keep the bits
// with count >= theta, store the token's word if asked, and OR the block's
// tokens into the window's word.
constexpr int VT = 1024;
constexpr int VTOK = VT / 64;  // tokens per block, one per wave

__global__ __launch_bounds__(VT) void vote_union_kernel(const GoldenArgs a) {
  __shared__ uint64_t part[VTOK][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t w = (int64_t)blockIdx.x * 64 + lane;
  const int tok = blockIdx.y * VTOK + wv;
  uint64_t g = 0;
  if (tok < a.T && w < a.W) {
    uint64_t c[7] = {0, 0, 0, 0, 0, 0, 0};
    const uint64_t* m = a.row_mask + (int64_t)tok * a.L * a.W + w;
    for (int l = 0; l < a.L; ++l) {
      uint64_t carry = m[(int64_t)l * a.W];
#pragma unroll
      for (int b = 0; b < 7; ++b) {
        const uint64_t nc = c[b] & carry;
        c[b] ^= carry;
        carry = nc;
      }
    }
    // count >= theta, most significant plane first
    uint64_t gt = 0, eq = ~0ull;
#pragma unroll
    for (int b = 6; b >= 0; --b) {
      if ((a.theta >> b) & 1) {
        eq &= c[b];
      } else {
        gt |= eq & c[b];
        eq &= ~c[b];
      }
    }
    g = gt | eq;
    if (a.token_golden) a.token_golden[(int64_t)tok * a.W + w] = g;
  }
  part[wv][lane] = g;
  __syncthreads();
  if (wv == 0 && w < a.W) {
    uint64_t u = 0;
#pragma unroll
    for (int j = 0; j < VTOK; ++j) u |= part[j][lane];
    if (u) atomicOr((unsigned long long*)&a.golden[w], (unsigned long long)u);
  }
}

}  // namespace

hipError_t launch_golden(const GoldenArgs& a, hipStream_t st) {
  const int rows = a.T * a.L;
  hipLaunchKernelGGL(nucleus_kernel, dim3(rows), dim3(GT), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 g((unsigned)((a.W + 63) / 64), (unsigned)((a.T + VTOK - 1) / VTOK));
  hipLaunchKernelGGL(vote_union_kernel, g, dim3(VT), 0, st, a);
  return hipGetLastError();
}

}  // namespace lsa
