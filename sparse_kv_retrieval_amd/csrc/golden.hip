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
// Four kernels, in order:
//
// 1. segment_kernel: one 512-thread block per segment (SEG entries) of a
//    (token, layer) row. It reads the logits once. Each lane keeps online
//    softmax statistics of its entries (its maximum m and the fp64 sum of
//    exp(y - m)). Each wave keeps its own list of the entries whose key is at
//    or above its filter, in its own LDS region, with a register count: pushes
//    need no atomics and no barriers. The first filter is the smallest of the
//    waves' second largest lane maxima over the first chunk; a wave whose list
//    passes half its region keeps its largest keys and raises its filter. The
//    segment's record (M, Z, the common filter, the entries at or above it)
//    goes to the workspace.
// 2. resolve_kernel: one 256-thread block per row. It merges the row's
//    segment records into an LDS list (every entry at or above the largest of
//    the segments' filters), buckets the list by distance below the row
//    maximum (fp64 masses), finds the bucket where the running mass crosses p,
//    ranks that bucket's entries exactly by (key descending, index ascending),
//    walks their masses to the crossing, and writes the row's mask. A row it
//    cannot finish that way (a list that overflowed or does not hold mass p, a
//    crowded crossing bucket) is appended to a list in the workspace.
// 3. fallback_kernel: a small grid over the rows resolve listed. A second read
//    builds a 4096-bin fp64 mass histogram over the top 12 key bits (LDS
//    atomics) and finds the crossing bin; a third read writes the mask bits of
//    the entries above it and lists the bin's entries; radix levels of 9, 9 and
//    2 bits over that list (or over the row, when the bin does not fit) find T,
//    and a count select over indices finds the cut among equal keys.
// 4. vote_union_kernel: per (token, mask word), a bit-sliced count of the
//    layers' mask bits in 7 bit planes, compared with theta plane by plane,
//    and OR-ed over the window's tokens.
#include <type_traits>

#include "kernels.hpp"

namespace lsa {

namespace {

constexpr int GT = 512;           // threads per nucleus block
constexpr int GW = GT / 64;       // waves per nucleus block
constexpr int GLL = 8;            // dword loads per lane per wave chunk
constexpr int GWC = 64 * GLL;     // entries per wave chunk: 8 mask words
constexpr int GBC = GWC * GW;     // entries per block chunk
constexpr int NB1 = 4096;         // fallback level-1 bins: key bits 31..20
constexpr int LB = 9;             // radix level width: one digit per thread
constexpr int NBL = 1 << LB;
constexpr int GCAP = 2048;        // entries held in the LDS list
constexpr int BOOT = 2;           // first filter: the smallest of the waves' BOOT-th largest lane maxima
constexpr int LW = GCAP / GW;     // list entries per wave in the segment kernel
constexpr int SEG = 32768;        // entries per row segment (one block of the first kernel)
constexpr uint32_t NONE = 0xFFFFFFFFu;
constexpr float LOG2E = 1.4426950408889634f;

// A segment's record in the workspace, followed by its list (key, index).
struct SegHead {
  double Z;         // sum of exp(y - M) over the segment
  float M;          // the segment's largest logit (-inf: empty)
  uint32_t tau;     // the list holds every entry of the segment whose key is >= tau
  uint32_t count;   // entries in the list
  uint32_t ovf;     // the list overflowed and is incomplete
  uint32_t pad[2];
};
constexpr int SEG_BYTES = (int)sizeof(SegHead) + GCAP * 8;

struct GoldenSmem {
  union {
    double bins[NB1];   // fallback level-1 masses (not live at the same time as the list)
    struct {
      uint32_t ckey[GCAP];  // the list
      uint32_t cidx[GCAP];
      struct {              // fast path: the entries of the crossing bucket, as listed and by rank
        uint32_t key[GT], idx[GT], rkey[GT], ridx[GT];
        double w[GT], rw[GT];
        uint32_t n;
      } cb;
    };
  };
  double lw[NBL];       // radix level weights
  uint32_t lc[NBL];     // radix level counts
  double wsum[GW];
  float wmax[GW], wmin[GW];
  uint32_t wu[GW], wo[GW];
  double res_A;
  uint32_t res_digit, res_cnt, ncand, kept, tau;
  int32_t last;
};

__device__ __forceinline__ float key_value(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// The smallest logit whose key is at or above the filter key tau (key 0: all).
// For finite y, key(y) >= tau iff y >= filter_value(tau).
__device__ __forceinline__ float filter_value(uint32_t tau) { return tau ? key_value(tau) : -INFINITY; }

// max of two finite floats (no NaN quieting: the inputs are finite logits)
__device__ __forceinline__ float fmax_finite(float a, float b) { return __builtin_amdgcn_fmed3f(a, b, INFINITY); }

// Unnormalised probability of a logit relative to a reference m >= y.
__device__ __forceinline__ float rel_mass(float y, float m) { return __builtin_amdgcn_exp2f((y - m) * LOG2E); }

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
// thread order, and the block total (NW waves; wsum is an NW-entry LDS table).
// excl of thread t + 1 equals incl of thread t bit for bit, so the running
// sums are exactly monotone.
template <int NW>
__device__ __forceinline__ void block_scan_f64_n(double v, double* wsum, double& excl, double& incl,
                                                 double& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  double x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  const double prev = __shfl_up(x, 1);
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  double off = 0.0, tot = 0.0;
  for (int i = 0; i < NW; ++i) {
    if (i == w) off = tot;
    tot += wsum[i];
  }
  __syncthreads();
  incl = off + x;
  excl = lane == 0 ? off : off + prev;
  total = tot;
}

__device__ __forceinline__ void block_scan_f64(double v, GoldenSmem& sm, double& excl, double& incl, double& total) {
  block_scan_f64_n<GW>(v, sm.wsum, excl, incl, total);
}

__device__ __forceinline__ double block_sum_f64(double v, GoldenSmem& sm) {
  double ex, in, tot;
  block_scan_f64(v, sm, ex, in, tot);
  return tot;
}

// sm.last = max(sm.last, the largest thread index where `has` holds): one LDS
// atomic per wave. Every thread of the block calls it.
__device__ __forceinline__ void note_last(GoldenSmem& sm, bool has) {
  const uint64_t m = __ballot(has);
  if ((threadIdx.x & 63) == 0 && m) atomicMax(&sm.last, (int32_t)(threadIdx.x + 63 - __builtin_clzll(m)));
}

// Where a radix level's items come from: the LDS list, or the whole row.
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

// The segment lists of one row, read from the workspace: one wave per segment,
// four entries per lane in flight. f runs in divergent lanes (no wave-wide ops).
struct FromSegs {
  const char* rec;
  uint32_t nseg;
  template <class F>
  __device__ __forceinline__ void each(F&& f) const {
    const uint32_t wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (uint32_t s = wv; s < nseg; s += GW) {
      const SegHead* h = (const SegHead*)(rec + (int64_t)s * SEG_BYTES);
      const uint32_t cnt = h->count;
      const uint2* lst = (const uint2*)(h + 1);
      for (uint32_t j0 = 0; j0 < cnt; j0 += 256) {
        uint2 e[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t j = j0 + 64u * u + lane;
          e[u] = j < cnt ? lst[j] : make_uint2(0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (j0 + 64u * u + lane < cnt) f(e[u].x, e[u].y);
      }
    }
  }
};

// One radix level. For each item, item(key, idx, rk, wt) says whether it takes
// part and gives its radix value rk and weight wt. Among the items whose rk
// has the prefix pre above bit sh + wb, the wb-bit digit at bit sh where the
// cumulative weight, taken from the largest digit down on top of A, reaches
// target. Returns the digit, A plus the weight above it, and its item count.
// When rounding leaves the sum short, the lowest digit holding items is taken.
template <class Src, class Item>
__device__ void radix_level(GoldenSmem& sm, const Src& src, const Item& item, uint32_t pre, int sh, int wb,
                            double target, double& A, uint32_t& digit, uint32_t& count) {
  const int t = threadIdx.x;
  const uint32_t nd = 1u << wb, dmask = nd - 1;
  __syncthreads();  // earlier readers of lw / lc are done
  sm.lw[t] = 0.0;
  sm.lc[t] = 0;
  if (t == 0) {
    sm.res_digit = NONE;
    sm.last = -1;
  }
  __syncthreads();
  src.each([&](uint32_t key, uint32_t idx) {
    uint32_t rk;
    double wt;
    if (item(key, idx, rk, wt) && (uint32_t)((uint64_t)rk >> (sh + wb)) == pre) {
      const uint32_t d = (rk >> sh) & dmask;
      lds_add(&sm.lw[d], wt);
      lds_inc(&sm.lc[d]);
    }
  });
  __syncthreads();
  const bool on = (uint32_t)t < nd;
  const uint32_t d = on ? nd - 1 - t : 0;  // thread order = descending digit
  const double m = on ? sm.lw[d] : 0.0;
  const uint32_t c = on ? sm.lc[d] : 0u;
  double ex, in, tot;
  block_scan_f64(m, sm, ex, in, tot);
  if (c > 0 && A + ex < target && A + in >= target) {
    sm.res_digit = d;
    sm.res_A = A + ex;
    sm.res_cnt = c;
  }
  note_last(sm, c > 0);
  __syncthreads();
  if (sm.res_digit != NONE) {
    digit = sm.res_digit;
    A = sm.res_A;
    count = sm.res_cnt;
  } else if (sm.last >= 0) {
    const uint32_t dl = nd - 1 - (uint32_t)sm.last;
    digit = dl;
    A = A + (tot - sm.lw[dl]);
    count = sm.lc[dl];
  } else {  // no item under the prefix (not reached: the prefix always holds an item)
    digit = 0;
    count = 0;
  }
}

// Radix select over the low `bits` bits of radix values whose higher bits are
// pre (levels of up to LB bits): the largest value v whose cumulative weight
// (items with rk >= v, on top of A) reaches target. A becomes A plus the
// weight of the items above v; cnt is the number of items equal to v.
template <class Src, class Item>
__device__ uint32_t radix_select(GoldenSmem& sm, const Src& src, const Item& item, double target, double& A,
                                 uint32_t& cnt, uint32_t pre = 0, int bits = 32) {
  uint32_t v = pre;
  while (bits > 0) {
    const int wb = bits < LB ? bits : LB;
    bits -= wb;
    uint32_t d;
    radix_level(sm, src, item, v, bits, wb, target, A, d, cnt);
    v = (v << wb) | d;
  }
  return v;
}

// Index cut among the nT entries whose key is T, given A, the mass of every
// entry above T: they share one mass w, and the j-th of them (by ascending
// index) is kept while A + (j - 1) w < target, so c = ceil((target - A) / w)
// of them are, at least one. Returns the largest kept index (all of them:
// 0x7FFFFFFF).
template <class Src>
__device__ uint32_t tie_cut(GoldenSmem& sm, const Src& src, uint32_t T, uint32_t nT, double A, double target,
                            float M) {
  const double w = (double)rel_mass(key_value(T), M);
  const double q = (target - A) / w;
  uint32_t c = nT;
  if (q < (double)nT) c = q <= 1.0 ? 1u : (uint32_t)ceil(q);
  if (c >= nT) return 0x7FFFFFFFu;
  double A2 = 0.0;
  uint32_t cc;
  const uint32_t r = radix_select(
      sm, src,
      [T](uint32_t key, uint32_t idx, uint32_t& rk, double& wt) {
        rk = ~idx;  // largest first = ascending index
        wt = 1.0;
        return key == T;
      },
      (double)c, A2, cc);
  return ~r;
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

// The same with two chunks in flight while one is processed (pass F, which
// has the registers for it); first(v) is called once on the first chunk.
template <class P, class F>
__device__ __forceinline__ void stream_row3(const __amdgpu_buffer_rsrc_t rs, uint32_t wv, uint32_t lane, uint32_t nit,
                                            P&& first, F&& body) {
  float va[GLL], vb[GLL], vc[GLL];
  auto off = [&](uint32_t it) { return ((it * GW + wv) * GWC + lane) * 4u; };
  load_chunk(rs, off(0), va);
  load_chunk(rs, off(1), vb);
  first(va);  // sees the first chunk while the second is in flight
  for (uint32_t it = 0;; it += 3) {
    load_chunk(rs, off(it + 2), vc);
    body(va, (it * GW + wv) * GWC);
    if (it + 1 >= nit) break;
    load_chunk(rs, off(it + 3), va);
    body(vb, ((it + 1) * GW + wv) * GWC);
    if (it + 2 >= nit) break;
    load_chunk(rs, off(it + 4), vb);
    body(vc, ((it + 2) * GW + wv) * GWC);
    if (it + 3 >= nit) break;
  }
}

// Appends (key, idx) to the LDS list for the lanes where `pass` holds (one LDS
// atomic per wave). Positions at or beyond GCAP are counted but not stored.
__device__ __forceinline__ void list_push(GoldenSmem& sm, bool pass, uint32_t key, uint32_t idx, uint32_t lane) {
  const uint64_t pm = __ballot(pass);
  if (pm) {
    uint32_t c0 = 0;
    if (lane == 0)
      c0 = __hip_atomic_fetch_add(&sm.ncand, (uint32_t)__popcll(pm), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    c0 = __shfl(c0, 0);
    if (pass) {
      const uint32_t pos = c0 + below(pm);
      if (pos < GCAP) {
        sm.ckey[pos] = key;
        sm.cidx[pos] = idx;
      }
    }
  }
}

// The R-th largest key (1 <= R <= m) among the m <= LW keys of a wave's list
// region: bit by bit from the top, the largest v with count(key >= v) >= R.
// Every lane of the wave calls it; no LDS writes.
__device__ uint32_t wave_kth_key(const uint32_t* keys, uint32_t m, uint32_t R, uint32_t lane) {
  uint32_t kk[LW / 64];
#pragma unroll
  for (int u = 0; u < LW / 64; ++u) {
    const uint32_t j = 64u * u + lane;
    kk[u] = j < m ? keys[j] : 0u;  // key 0 is below every candidate value tried
  }
  uint32_t v = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = v | (1u << b);
    uint32_t cnt = 0;
#pragma unroll
    for (int u = 0; u < LW / 64; ++u) cnt += (uint32_t)__popcll(__ballot(kk[u] >= c));
    if (cnt >= R) v = c;
  }
  return v;
}

// The rows the resolve kernel leaves to the fallback, after the segment records in the
// workspace: a count (cleared by the segment kernel), then the rows in any order.
__device__ __forceinline__ uint32_t* fallback_count(const GoldenArgs& a) {
  return (uint32_t*)(a.ws + (int64_t)a.T * a.L * a.S * SEG_BYTES);
}
__device__ __forceinline__ uint32_t* fallback_rows(const GoldenArgs& a) { return fallback_count(a) + 1; }

// Kernel 1: one block per segment of SEG entries of a (token, layer) row.
// Each wave keeps its own part of the list (LW entries of LDS, a register
// count, its own filter), so pushes need no atomics and no barriers.
struct SegSmem {
  uint32_t ckey[GCAP];
  uint32_t cidx[GCAP];
  double wsum[GW];
  float wmax[GW], wmin[GW];
  uint32_t wu[GW], wo[GW];
};

__global__ __launch_bounds__(GT) __attribute__((amdgpu_waves_per_eu(6, 6)))
void segment_kernel(const GoldenArgs a) {
  __shared__ SegSmem sm;
  const int t = threadIdx.x;
  const uint32_t wv = uni((int32_t)(t >> 6));  // wave-uniform
  const uint32_t lane = t & 63;
  const int row = blockIdx.y, seg = blockIdx.x;
  // the fallback list starts empty (the resolve kernel, next on the stream, appends to it)
  if (row == 0 && seg == 0 && t == 0) *fallback_count(a) = 0u;
  const int tok = row / a.L;
  const int32_t nv = a.n_valid[tok];
  const uint32_t nrow = (uint32_t)min((int64_t)max(nv, 0), a.row_stride);
  const uint32_t s0 = (uint32_t)seg * SEG;
  SegHead* h = (SegHead*)(a.ws + ((int64_t)row * a.S + seg) * SEG_BYTES);
  uint2* lst = (uint2*)(h + 1);
  if (s0 >= nrow) {
    if (t == 0) *h = SegHead{0.0, -INFINITY, 0u, 0u, 0u, {0u, 0u}};
    return;
  }
  const uint32_t n = min(nrow - s0, (uint32_t)SEG);  // entries of this segment
  const auto rs = buf_rsrc(a.logits + (int64_t)row * a.row_stride + s0, n * 4u);
  const uint32_t nit = (n + GBC - 1) / GBC;
  uint32_t* wkey = sm.ckey + wv * LW;
  uint32_t* widx = sm.cidx + wv * LW;

  float ml = -INFINITY;  // this lane's maximum and sum of exp(y - ml)
  double sl = 0.0;
  uint32_t wc = 0;       // entries in this wave's list (wave-uniform)
  bool wovf = false;     // this wave's list overflowed (wave-uniform)
  float tauf = -INFINITY;  // this wave's filter: its list holds every entry it saw at or above it
  auto first = [&](float (&v)[GLL]) {
    // First filter: every wave's BOOT-th largest lane maximum over its first
    // chunk, and the smallest of those (one wave's sample alone can sit high).
    float x = -INFINITY, kth = -INFINITY;
#pragma unroll
    for (int k = 0; k < GLL; ++k)
      if (wv * GWC + 64u * k + lane < n) x = fmaxf(x, v[k]);
    for (int r = 0; r < BOOT; ++r) {
      float m = x;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
      kth = m;
      const uint64_t at = __ballot(x == m);
      if (lane == (uint32_t)__builtin_ctzll(at)) x = -INFINITY;
    }
    if (lane == 0) sm.wmin[wv] = kth == -INFINITY ? INFINITY : kth;  // a wave without entries has no say
    __syncthreads();
    float f = INFINITY;
#pragma unroll
    for (int j = 0; j < GW; ++j) f = fminf(f, sm.wmin[j]);
    tauf = f == INFINITY ? -INFINITY : f;
  };
  // One chunk: lane statistics and list pushes. FULL: every entry is inside the
  // segment (all chunks but the last), so no per-entry bounds test.
  auto chunk = [&](auto full_t, float (&v)[GLL], uint32_t base) {
    constexpr bool FULL = decltype(full_t)::value;
    bool ok[GLL];
#pragma unroll
    for (int k = 0; k < GLL; ++k) ok[k] = FULL || base + 64u * k + lane < n;
    float cm = ml;
#pragma unroll
    for (int k = 0; k < GLL; ++k) cm = ok[k] ? fmax_finite(cm, v[k]) : cm;
    // rescale the running sum when the maximum grows (the factor is 1 otherwise)
    const float f = cm == ml ? 1.f : rel_mass(ml, cm);  // 0 while ml is still -inf
    ml = cm;
    float ps = 0.f;
#pragma unroll
    for (int k = 0; k < GLL; ++k) {
      const float e = rel_mass(v[k], ml);
      ps += FULL ? e : (ok[k] ? e : 0.f);
    }
    sl = sl * (double)f + (double)ps;
    // entries at or above the filter go to the wave's list
    uint64_t pm[GLL];
    uint32_t tot = 0;
#pragma unroll
    for (int k = 0; k < GLL; ++k) {
      pm[k] = __ballot(ok[k] & (v[k] >= tauf));
      tot += (uint32_t)__popcll(pm[k]);
    }
    if (tot) {
      uint32_t pos = wc;
#pragma unroll
      for (int k = 0; k < GLL; ++k) {
        if (pm[k]) {  // most loads of a chunk have no entry above the filter
          const uint32_t p = pos + below(pm[k]);
          if (((pm[k] >> lane) & 1) && p < (uint32_t)LW) {
            wkey[p] = order_key(v[k]);
            widx[p] = s0 + base + 64u * k + lane;
          }
          pos += (uint32_t)__popcll(pm[k]);
        }
      }
      wc = pos;
      if (wc > (uint32_t)LW) {  // entries were lost: the row takes the fallback
        wovf = true;
        tauf = INFINITY;
      } else if (wc > (uint32_t)LW / 2) {
        // keep the LW / 4 largest keys (and their ties) and raise the filter to the smallest of them
        const uint32_t kv = wave_kth_key(wkey, wc, LW / 4, lane);
        uint32_t kk[LW / 64], xx[LW / 64];
#pragma unroll
        for (int u = 0; u < LW / 64; ++u) {
          const uint32_t j = 64u * u + lane;
          kk[u] = j < wc ? wkey[j] : 0u;
          xx[u] = j < wc ? widx[j] : 0u;
        }
        uint32_t q = 0;
#pragma unroll
        for (int u = 0; u < LW / 64; ++u) {
          const uint64_t km = __ballot(kk[u] >= kv);
          if ((km >> lane) & 1) {
            wkey[q + below(km)] = kk[u];
            widx[q + below(km)] = xx[u];
          }
          q += (uint32_t)__popcll(km);
        }
        wc = q;
        tauf = key_value(kv);
      }
    }
  };
  stream_row3(rs, wv, lane, nit, first, [&](float (&v)[GLL], uint32_t base) {
    if (base + GWC <= n)
      chunk(std::true_type{}, v, base);
    else
      chunk(std::false_type{}, v, base);
  });

  // ---- the segment's M, Z and common filter, then its record
  float wm = ml;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) wm = fmaxf(wm, __shfl_xor(wm, o));
  if (lane == 0) {
    sm.wmax[wv] = wm;
    sm.wu[wv] = tauf == -INFINITY ? 0u : (wovf ? 0xFFFFFFFFu : order_key(tauf));
    sm.wo[wv] = wovf ? 1u : 0u;
  }
  __syncthreads();
  float M = -INFINITY;
  uint32_t tau = 0;
  bool ovf = false;
#pragma unroll
  for (int j = 0; j < GW; ++j) {
    M = fmaxf(M, sm.wmax[j]);
    tau = max(tau, sm.wu[j]);
    ovf = ovf || sm.wo[j];
  }
  double ex, in, Z;
  block_scan_f64_n<GW>(ml == -INFINITY ? 0.0 : sl * (double)rel_mass(ml, M), sm.wsum, ex, in, Z);
  // every wave's list is complete at or above its own filter, so all are at or above tau
  uint32_t kk[LW / 64], xx[LW / 64], mine = 0;
  uint64_t km[LW / 64];
#pragma unroll
  for (int u = 0; u < LW / 64; ++u) {
    const uint32_t j = 64u * u + lane;
    kk[u] = j < wc ? wkey[j] : 0u;
    xx[u] = j < wc ? widx[j] : 0u;
    km[u] = __ballot(!ovf && j < wc && kk[u] >= tau);
    mine += (uint32_t)__popcll(km[u]);
  }
  if (lane == 0) sm.wu[wv] = mine;
  __syncthreads();
  uint32_t off = 0, cnt = 0;
#pragma unroll
  for (int j = 0; j < GW; ++j) {
    off += j < (int)wv ? sm.wu[j] : 0u;
    cnt += sm.wu[j];
  }
#pragma unroll
  for (int u = 0; u < LW / 64; ++u) {
    if ((km[u] >> lane) & 1) lst[off + below(km[u])] = make_uint2(kk[u], xx[u]);
    off += (uint32_t)__popcll(km[u]);
  }
  if (t == 0) *h = SegHead{Z, M, tau, cnt, ovf ? 1u : 0u, {0u, 0u}};
}

// Kernel 2: one 256-thread block per (token, layer) row. Merges the row's
// segment records into an LDS list (every entry at or above the largest of the
// segments' filters), finds the crossing bucket of the mass by distance below
// M, ranks that bucket's entries exactly, and writes the row's mask. A row it
// cannot finish that way (a list that overflowed or does not hold mass p, a
// crowded bucket) is listed for the fallback kernel.
constexpr int RT = 256;           // threads per resolve block
constexpr int RW = RT / 64;
constexpr int NBR = RT;           // buckets: one per thread
constexpr int MCAP = 2048;        // merged list entries held in LDS
constexpr int CBR = 128;          // entries of the crossing bucket ranked in LDS

struct ResolveSmem {
  uint32_t key[MCAP], idx[MCAP];
  double lw[NBR];
  uint32_t lc[NBR];
  uint32_t soff[RT + 1];
  struct {
    uint32_t key[CBR], idx[CBR], rkey[CBR], ridx[CBR];
    double w[CBR], rw[CBR];
    uint32_t n;
  } cb;
  double wsum[RW];
  float wmax[RW];
  uint32_t wu[RW], wo[RW];
  double res_A;
  uint32_t res_digit, res_cnt;
  int32_t last;
};

__global__ __launch_bounds__(RT) void resolve_kernel(const GoldenArgs a) {
  __shared__ ResolveSmem sm;
  const int t = threadIdx.x;
  const uint32_t wv = uni((int32_t)(t >> 6));  // wave-uniform
  const uint32_t lane = t & 63;
  const int row = blockIdx.x;
  const int tok = row / a.L;
  const int32_t nv = a.n_valid[tok];
  const uint32_t n = (uint32_t)min((int64_t)max(nv, 0), a.row_stride);
  const uint32_t nw = (n + 63) >> 6;
  uint64_t* words = a.row_mask + (int64_t)row * a.W;

  if (row == 0)
    for (int64_t j = t; j < a.W; j += RT) a.golden[j] = 0;  // the vote kernel ORs into it
  for (uint32_t j = nw + t; j < (uint32_t)a.W; j += RT) words[j] = 0;
  if (n == 0) {
    if (t == 0 && a.nucleus_size) a.nucleus_size[row] = 0;
    return;
  }

  // ---- the segment records: M, Z, the common filter, the list offsets
  const uint32_t nseg = (n + SEG - 1) / SEG;
  const char* rec = a.ws + (int64_t)row * a.S * SEG_BYTES;
  float hm = -INFINITY;
  double hz = 0.0;
  uint32_t ht = 0, hc = 0, ho = 0;
  if ((uint32_t)t < nseg) {  // one record per thread; longer rows take the fallback
    const SegHead* h = (const SegHead*)(rec + (int64_t)t * SEG_BYTES);
    hm = h->M;
    hz = h->Z;
    ht = h->tau;
    hc = h->count;
    ho = h->ovf;
  }
  {
    float m = hm;
    uint32_t tm = ht, o = ho;
#pragma unroll
    for (int x = 32; x > 0; x >>= 1) {
      m = fmaxf(m, __shfl_xor(m, x));
      tm = max(tm, (uint32_t)__shfl_xor((int)tm, x));
      o |= (uint32_t)__shfl_xor((int)o, x);
    }
    if (lane == 0) {
      sm.wmax[wv] = m;
      sm.wu[wv] = tm;
      sm.wo[wv] = o;
    }
  }
  __syncthreads();
  float M = -INFINITY;
  uint32_t tau = 0;
  bool fb = nseg >= (uint32_t)RT;
#pragma unroll
  for (int j = 0; j < RW; ++j) {
    M = fmaxf(M, sm.wmax[j]);
    tau = max(tau, sm.wu[j]);
    fb = fb || sm.wo[j];
  }
  double ex, in, tot;
  block_scan_f64_n<RW>(hm == -INFINITY ? 0.0 : hz * (double)rel_mass(hm, M), sm.wsum, ex, in, tot);
  const double target = (double)a.p * tot;
  block_scan_f64_n<RW>((double)hc, sm.wsum, ex, in, tot);  // list counts: exact in fp64
  if ((uint32_t)t <= nseg) sm.soff[t] = (uint32_t)ex;       // soff[nseg]: the total
  const uint32_t total = (uint32_t)tot;
  fb = fb || total > (uint32_t)MCAP;
  uint32_t kept = 0;
  if (!fb) {
    __syncthreads();
    // gather the lists (every entry with key >= tau is in them: tau is at or
    // above each segment's filter)
    for (uint32_t g0 = 0; g0 < total; g0 += 4 * RT) {
      uint2 e[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t g = g0 + u * RT + t;
        e[u] = make_uint2(0u, 0u);
        if (g < total) {
          uint32_t sg = 0;
          while (sm.soff[sg + 1] <= g) ++sg;
          e[u] = ((const uint2*)(rec + (int64_t)sg * SEG_BYTES + sizeof(SegHead)))[g - sm.soff[sg]];
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t g = g0 + u * RT + t;
        if (g < total) {
          sm.key[g] = e[u].x;
          sm.idx[g] = e[u].y;
        }
      }
    }
    // buckets by distance below M over [lo, M]: ascending d is descending y
    float lo = filter_value(tau);
    if (tau == 0) {  // the lists hold the whole (short) row: its own minimum
      lo = INFINITY;
      for (uint32_t j = t; j < total; j += RT) lo = fminf(lo, key_value(sm.key[j]));
      __syncthreads();
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) lo = fminf(lo, __shfl_xor(lo, o));
      if (lane == 0) sm.wmax[wv] = lo;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < RW; ++j) lo = fminf(lo, sm.wmax[j]);
    }
    const float sc = M > lo ? (float)(NBR - 1) / (M - lo) : 0.f;
    auto bucket = [M, sc](float yv) { return (uint32_t)fminf((M - yv) * sc, (float)(NBR - 1)); };
    sm.lw[t] = 0.0;
    sm.lc[t] = 0;
    if (t == 0) {
      sm.res_digit = NONE;
      sm.last = -1;
      sm.cb.n = 0;
    }
    __syncthreads();
    for (uint32_t j = t; j < total; j += RT) {
      const uint32_t key = sm.key[j];
      if (key >= tau) {
        const float yv = key_value(key);
        const uint32_t d = bucket(yv);
        lds_add(&sm.lw[d], (double)rel_mass(yv, M));
        lds_inc(&sm.lc[d]);
      }
    }
    __syncthreads();
    const uint32_t c = sm.lc[t];
    block_scan_f64_n<RW>(sm.lw[t], sm.wsum, ex, in, tot);  // tot: the lists' mass at or above tau
    if (c > 0 && ex < target && in >= target) {
      sm.res_digit = t;
      sm.res_A = ex;
      sm.res_cnt = c;
    }
    {
      const uint64_t m = __ballot(c > 0);
      if (lane == 0 && m) atomicMax(&sm.last, (int32_t)(t + 63 - __builtin_clzll(m)));
    }
    __syncthreads();
    fb = !(tot > target * (1.0 + 1e-9));  // the nucleus does not lie inside the lists
    uint32_t db = 0, cnt = 0;
    double A = 0.0;
    if (!fb) {
      if (sm.res_digit != NONE) {
        db = sm.res_digit;
        A = sm.res_A;
        cnt = sm.res_cnt;
      } else {  // rounding left the sum short: the last bucket that holds entries
        db = (uint32_t)sm.last;
        A = tot - sm.lw[db];
        cnt = sm.lc[db];
      }
      fb = cnt > (uint32_t)CBR;
    }
    if (!fb) {
      // exact order inside the bucket: rank by (key descending, index ascending)
      for (uint32_t j = t; j < total; j += RT) {
        const uint32_t key = sm.key[j];
        if (key >= tau && bucket(key_value(key)) == db) {
          const uint32_t q = atomicAdd(&sm.cb.n, 1u);
          sm.cb.key[q] = key;
          sm.cb.idx[q] = sm.idx[j];
          sm.cb.w[q] = (double)rel_mass(key_value(key), M);
        }
      }
      __syncthreads();
      if ((uint32_t)t < cnt) {
        const uint32_t kt = sm.cb.key[t], it2 = sm.cb.idx[t];
        uint32_t r = 0;
        for (uint32_t j = 0; j < cnt; ++j) {
          const uint32_t kj = sm.cb.key[j];
          r += (kj > kt || (kj == kt && sm.cb.idx[j] < it2)) ? 1u : 0u;
        }
        sm.cb.rkey[r] = kt;
        sm.cb.ridx[r] = it2;
        sm.cb.rw[r] = sm.cb.w[t];
      }
      __syncthreads();
      // kept while the mass before it is below the target; rank 0 always is
      block_scan_f64_n<RW>((uint32_t)t < cnt ? sm.cb.rw[t] : 0.0, sm.wsum, ex, in, tot);
      const bool keep = (uint32_t)t < cnt && (t == 0 || A + ex < target);
      const bool next = (uint32_t)t + 1 < cnt && A + in < target;
      if (keep && !next) {
        sm.res_digit = sm.cb.rkey[t];
        sm.res_cnt = sm.cb.ridx[t];
      }
      __syncthreads();
      const uint32_t T = sm.res_digit, ncut = sm.res_cnt;
      for (uint32_t j = t; j < nw; j += RT) words[j] = 0;
      // the cleared words are stored before any wave's bit below (one L2 for the block)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __syncthreads();
      for (uint32_t j = t; j < total; j += RT) {
        const uint32_t key = sm.key[j], idx = sm.idx[j];
        if (key > T || (key == T && idx <= ncut)) {  // T >= tau: these are at or above the filter
          __hip_atomic_fetch_or(&words[idx >> 6], (uint64_t)1 << (idx & 63), __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_WORKGROUP);
          ++kept;
        }
      }
    }
  }
  if (t == 0 && fb) fallback_rows(a)[atomicAdd(fallback_count(a), 1u)] = (uint32_t)row;
  if (!fb && a.nucleus_size) {
    block_scan_f64_n<RW>((double)kept, sm.wsum, ex, in, tot);
    if (t == 0) a.nucleus_size[row] = (int32_t)tot;
  }
}

// Kernel 3: the fallback, for the rows the resolve kernel listed. M comes from
// the segment records again. One row at a time per block.
__device__ __forceinline__ void fallback_row(const GoldenArgs& a, const int row, GoldenSmem& sm) {
  const int t = threadIdx.x;
  const uint32_t wv = uni((int32_t)(t >> 6));  // wave-uniform
  const uint32_t lane = t & 63;
  const int tok = row / a.L;
  const int32_t nv = a.n_valid[tok];
  const uint32_t n = (uint32_t)min((int64_t)max(nv, 0), a.row_stride);
  const uint32_t nw = (n + 63) >> 6;
  const float* y = a.logits + (int64_t)row * a.row_stride;
  uint64_t* words = a.row_mask + (int64_t)row * a.W;
  const auto rs = buf_rsrc(y, n * 4u);
  const uint32_t nit = (n + GBC - 1) / GBC;

  if (n == 0) return;

  // ---- the row maximum from the segment records
  const uint32_t nseg = (n + SEG - 1) / SEG;
  const char* rec = a.ws + (int64_t)row * a.S * SEG_BYTES;
  float M = -INFINITY;
  for (uint32_t s = t; s < nseg; s += GT) M = fmaxf(M, ((const SegHead*)(rec + (int64_t)s * SEG_BYTES))->M);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  if (lane == 0) sm.wmax[wv] = M;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < GW; ++j) M = fmaxf(M, sm.wmax[j]);
  uint32_t kept = 0;
  {
    // ---- fallback: level-1 mass histogram (second read; M is known now)
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NB1 / GT; ++j) sm.bins[t * (NB1 / GT) + j] = 0.0;
    if (t == 0) sm.ncand = 0;
    __syncthreads();
    stream_row(rs, wv, lane, nit, [&](float (&v)[GLL], uint32_t base) {
      if (base + GWC <= n) {
#pragma unroll
        for (int k = 0; k < GLL; ++k) lds_add(&sm.bins[order_key(v[k]) >> 20], (double)rel_mass(v[k], M));
      } else {
#pragma unroll
        for (int k = 0; k < GLL; ++k)
          if (base + 64u * k + lane < n) lds_add(&sm.bins[order_key(v[k]) >> 20], (double)rel_mass(v[k], M));
      }
    });
    __syncthreads();

    // crossing bin b1 of the cumulative mass at p * Zh, Zh the histogram total
    double A, tgt;
    uint32_t b1;
    {
      double l[NB1 / GT], s = 0.0;  // this thread's bins, descending
#pragma unroll
      for (int j = 0; j < NB1 / GT; ++j) {
        s += sm.bins[NB1 - 1 - (NB1 / GT) * t - j];
        l[j] = s;
      }
      double ex, in, Zh;
      block_scan_f64(s, sm, ex, in, Zh);
      tgt = (double)a.p * Zh;
      if (t == 0) sm.res_digit = NONE;
      __syncthreads();
      if (ex < tgt && in >= tgt) {
        // first of this thread's bins whose running sum reaches the target;
        // if rounding leaves it short, the last bin that holds mass
        int jj = -1, jm = 0;
        double above = ex, above_m = ex, prev = 0.0;
#pragma unroll
        for (int j = 0; j < NB1 / GT; ++j) {
          if (jj < 0 && ex + l[j] >= tgt) {
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

    // mask words for the entries outside b1, list of the entries in b1 (third read)
    stream_row(rs, wv, lane, nit, [&](float (&v)[GLL], uint32_t base) {
      uint64_t mine = 0;
#pragma unroll
      for (int k = 0; k < GLL; ++k) {
        const uint32_t e = base + 64u * k + lane;
        const uint32_t key = order_key(v[k]);
        const bool valid = e < n;
        const uint64_t kw = __ballot(valid && (key >> 20) > b1);
        if (lane == 0) kept += (uint32_t)__popcll(kw);  // counted once per wave
        mine = lane == (uint32_t)k ? kw : mine;
        list_push(sm, valid && (key >> 20) == b1, key, e, lane);
      }
      const uint32_t wi = (base >> 6) + lane;
      if (lane < GLL && wi < nw) words[wi] = mine;
    });
    // the mask stores are complete before any wave's fix-up atomic below
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    const uint32_t nc = sm.ncand;

    auto mass_item = [M](uint32_t key, uint32_t, uint32_t& rk, double& wt) {
      rk = key;
      wt = (double)rel_mass(key_value(key), M);
      return true;
    };
    uint32_t T, ncut;
    auto resolve = [&](const auto& src) {
      uint32_t nT;
      T = radix_select(sm, src, mass_item, tgt, A, nT, b1, 20);
      ncut = tie_cut(sm, src, T, nT, A, tgt, M);
    };
    if (nc <= GCAP) {
      resolve(FromList{&sm, nc});
      for (uint32_t j = t; j < nc; j += GT) {
        const uint32_t key = sm.ckey[j], idx = sm.cidx[j];
        if (key > T || (key == T && idx <= ncut)) {
          __hip_atomic_fetch_or(&words[idx >> 6], (uint64_t)1 << (idx & 63), __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_WORKGROUP);
          ++kept;
        }
      }
    } else {
      resolve(FromRow{rs, n});
      // rewrite every word; each word is stored by the same lane that stored it above
      kept = 0;
      stream_row(rs, wv, lane, nit, [&](float (&v)[GLL], uint32_t base) {
        uint64_t mine = 0;
#pragma unroll
        for (int k = 0; k < GLL; ++k) {
          const uint32_t e = base + 64u * k + lane;
          const uint32_t key = order_key(v[k]);
          const uint64_t kw = __ballot(e < n && (key > T || (key == T && e <= ncut)));
          if (lane == 0) kept += (uint32_t)__popcll(kw);
          mine = lane == (uint32_t)k ? kw : mine;
        }
        const uint32_t wi = (base >> 6) + lane;
        if (lane < GLL && wi < nw) words[wi] = mine;
      });
    }
  }
  if (a.nucleus_size) {
    const double tot = block_sum_f64((double)kept, sm);
    if (t == 0) a.nucleus_size[row] = (int32_t)tot;
  }
}

// A small grid walks the list (empty on most calls, so the launch costs little).
constexpr int FB_BLOCKS = 256;
__global__ __launch_bounds__(GT) void fallback_kernel(const GoldenArgs a) {
  __shared__ GoldenSmem sm;
  const uint32_t nf = *fallback_count(a);
  for (uint32_t i = blockIdx.x; i < nf; i += gridDim.x) {
    fallback_row(a, (int)fallback_rows(a)[i], sm);
    __syncthreads();  // the next row reuses sm
  }
}

// Per (token, word): count the L layers' bits in 7 bit planes, keep the bits
// with count >= theta, store the token's word if asked, and OR the block's
// tokens into the window's word.
constexpr int VT = 256;
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
    for (int l0 = 0; l0 < a.L; l0 += 8) {
      uint64_t x[8];  // eight layers' loads in flight at once
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = l0 + j < a.L ? m[(int64_t)(l0 + j) * a.W] : 0ull;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint64_t carry = x[j];
#pragma unroll
        for (int b = 0; b < 7; ++b) {
          const uint64_t nc = c[b] & carry;
          c[b] ^= carry;
          carry = nc;
        }
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

size_t golden_workspace_bytes(int64_t rows, int64_t row_stride) {
  // segment records, then the fallback list: its count and up to one entry per row
  return (size_t)rows * (size_t)((row_stride + SEG - 1) / SEG) * (size_t)SEG_BYTES + (size_t)(rows + 1) * 4;
}

hipError_t launch_golden(const GoldenArgs& a0, hipStream_t st) {
  GoldenArgs a = a0;
  a.S = (int32_t)((a.row_stride + SEG - 1) / SEG);
  const int rows = a.T * a.L;
  hipLaunchKernelGGL(segment_kernel, dim3((unsigned)a.S, (unsigned)rows), dim3(GT), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(resolve_kernel, dim3(rows), dim3(RT), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fallback_kernel, dim3((unsigned)std::min(rows, FB_BLOCKS)), dim3(GT), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 g((unsigned)((a.W + 63) / 64), (unsigned)((a.T + VTOK - 1) / VTOK));
  hipLaunchKernelGGL(vote_union_kernel, g, dim3(VT), 0, st, a);
  return hipGetLastError();
}

}  // namespace lsa
