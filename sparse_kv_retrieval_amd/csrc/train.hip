// One training step of a memory-indexer layer: loss and gradients of W^DQ,
// W^IUQ and W^w against frozen keys.
//
// marsggbo write-up, "4. 训练" (training), and the hyper.ai digest, "方法"
// (Method): the compressed index keys are precomputed and fixed, and only the
// query side's projections are trained, with binary cross-entropy made focal
// (the gist.science summary states the same loss). The score is the
// selection path's: I_s = sigmoid(x_s), x_s = sum_j w_j ReLU(q_j . K_s),
// q = (h W^DQ) W^IUQ, w = h W^w (the write-up's §3.1). Focal form with
// p = I_s: -alpha (1-p)^gamma log p for a golden entry, -(1-alpha) p^gamma
// log(1-p) otherwise; the loss is the mean over the batch's entries.
//
// Kernels, after a zero fill of c, q, w and the two projection stages (each
// reduction split over two blocks that add into the zeroed outputs):
//   train_scan_kernel  one pass over the keys. 4 waves per block, 16 heads per
//                      wave; the grid is one round of resident blocks, each a
//                      run of 32-entry tiles of one sequence. Each tile is
//                      staged in LDS twice (double-buffered): row-major for the
//                      score MFMAs, transposed for the gradient MFMAs. Per
//                      tile: the head dots S = K q^T on bf16 MFMA (q split
//                      hi + lo), x_s, the loss and g_s = d loss / d x_s, and
//                      the gradient contraction on MFMA with the gate factored
//                      out: dq'_j = sum_s g_s [S_sj > 0] K_s, with g_s split
//                      hi + lo once per entry. dq_j = w_j dq'_j and
//                      dw_j = sum_s g_s ReLU(S_sj) = q_j . dq'_j follow after
//                      the scan. The focal terms are evaluated once per entry
//                      in each wave and shared through LDS. Per-block partial
//                      sums (dq' and the loss) go to the workspace.
//   train_reduce_kernel  sums a sequence's block partials into dq' (one block per
//                      head and sequence) and forms dq and dw; one block sums
//                      the loss over every block.
//   train_dc_kernel    dc = dq W^IUQ (bf16 weights) in row slices of 128, each
//                      block one slice x 256 columns, and
//   train_sum_kernel   the slices' partials added.
//   train_outer_kernel rank-B products for the three gradients (16-byte stores):
//                      g_iuq = dq^T c; g_dq = dc^T h and g_w = dw^T h in one
//                      launch.
#include <algorithm>

#include "kernels.hpp"

namespace lsa {

namespace {

constexpr int TT = 256;            // scan block: 4 waves
constexpr int TNH = 64;            // heads (16 per wave)
constexpr int TDH = 128;           // head dim = key dim
constexpr int TE = 32;             // entries per tile
constexpr int SCAN_BLOCKS = 768;   // target grid: three resident blocks on each of 256 CUs, one round
constexpr int MIN_TPB = 8;         // at least this many tiles per scan block
constexpr int PW = TNH * TDH + 1;  // floats per block partial: dq' (below) and the loss

// The transposed tile holds, for each key dim d, the tile's 32 entries in "slot" order: entry
// e = 16 mb + 4 kg + i sits in slot 8 kg + 4 mb + i, so that the gradient MFMA's k-group kg is
// exactly the entries whose head dots lane (head, kg) holds after the score MFMA. Row d is 64
// bytes (4 chunks of 8 slots); chunk c is stored at c ^ swz(d), which keeps both the paired
// writes and the MFMA reads free of LDS bank conflicts beyond two-way.
__device__ __forceinline__ int tt_swz(int d) { return ((d >> 2) ^ (d >> 4)) & 3; }
__device__ __forceinline__ int tt_slot(int e) { return 8 * ((e >> 2) & 3) + 4 * (e >> 4) + (e & 3); }

struct TrainScanSmem {
  uint4 kt[2][TE * 16];            // row-major tiles: chunk c of entry e at e*16 + (c ^ (e & 15))
  uint4 ktt[2][TDH * TE / 8];      // transposed tiles (above)
  float4 xpart[2][TE];             // per entry: the four waves' partial logits
  uint16_t gh[4][TE], gl[4][TE];   // per wave: d loss / d x of the tile's entries as bf16 hi + lo
  double lsum[4];
};

// log(1 + e) for e in [0, 1]: log(u) e / (u - 1) with u = 1 + e rounded, which cancels the rounding of u
// (Goldberg's form), so a hardware logarithm keeps a few-ulp relative error even for tiny e.
__device__ __forceinline__ float t_log1p(float e) {
  const float u = 1.f + e;
  return u == 1.f ? e : __logf(u) * (e * __builtin_amdgcn_rcpf(u - 1.f));
}

// Focal loss term and its derivative in the logit x (fp32), label y. With L = log(1 + e^-|x|),
// log p = min(x, 0) - L and log(1 - p) = min(-x, 0) - L; powers are exponentials of gamma times those.
__device__ __forceinline__ void focal(float x, bool y, float gamma, float alpha, float& loss, float& grad) {
  const float L = t_log1p(__expf(-fabsf(x)));
  const float lp = fminf(x, 0.f) - L, lq = fminf(-x, 0.f) - L;  // log p, log(1 - p)
  const float p = __expf(lp), q = __expf(lq);
  const float pw = __expf(gamma * (y ? lq : lp));                 // (1-p)^gamma or p^gamma
  if (y) {
    loss = -alpha * pw * lp;
    grad = alpha * pw * (gamma * p * lp - q);
  } else {
    loss = -(1.f - alpha) * pw * lq;
    grad = (1.f - alpha) * pw * (p - gamma * q * lq);
  }
}

// Two fp32 values to packed bf16 with the hardware's round-to-nearest-even conversion.
typedef __bf16 tbf16x2 __attribute__((ext_vector_type(2)));
typedef float tf32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((tf32x2){a, b}, tbf16x2));
}
// First scan block of sequence b (blocks are laid out sequence by sequence).
__device__ __forceinline__ int64_t first_block(const int64_t* __restrict__ off, int b, int64_t be) {
  int64_t s = 0;
  for (int i = 0; i < b; ++i) s += (off[i + 1] - off[i] + be - 1) / be;
  return s;
}

template <int N>
__device__ __forceinline__ float ror(float v) {  // lane i of each row of 16 gets lane (i + N) % 16
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x120 | N, 0xF, 0xF, true));
}
template <int N>
__device__ __forceinline__ uint32_t ror_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x120 | N, 0xF, 0xF, false);
}

__global__ __launch_bounds__(TT) void train_scan_kernel(const TrainArgs a) {
  __shared__ TrainScanSmem sm;
  const int t = threadIdx.x, lane = t & 63;
  const int wq = __builtin_amdgcn_readfirstlane(t >> 6);
  const int hl = lane & 15, kg = lane >> 4;
  // this block's sequence and entry range (blocks of a.tpb tiles, sequence by sequence)
  const int64_t be = (int64_t)a.tpb * TE;
  int b = 0;
  int64_t blk0 = 0;
  for (;; ++b) {
    const int64_t nb = (a.key_off[b + 1] - a.key_off[b] + be - 1) / be;
    if ((int64_t)blockIdx.x < blk0 + nb) break;
    blk0 += nb;
  }
  const int64_t n_b = a.key_off[b + 1] - a.key_off[b];
  const int64_t e_begin = ((int64_t)blockIdx.x - blk0) * be;
  const int ntiles = (int)min((int64_t)a.tpb, (n_b - e_begin + TE - 1) / TE);
  const auto rs = buf_rsrc((const char*)a.keys + a.key_off[b] * (TDH * 2), (uint32_t)(n_b * (TDH * 2)));
  const uint64_t* lab = a.labels + a.mwo[b];

  // this wave's 16 heads: q split into bf16 hi + lo (B operand of the score MFMA), and the gate
  const float* qrow = a.q + ((int64_t)b * TNH + 16 * wq + hl) * TDH;
  bf16x8 qh[4], ql[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = qrow[32 * ks + 8 * kg + j];
    split8(x, qh[ks], ql[ks]);
  }
  const float wh = a.w[(int64_t)b * TNH + 16 * wq + hl];

  f32x4 accb[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) accb[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  double ll = 0.0;

  // tile loads: thread t holds chunks 2g, 2g+1 (key dims 16g .. 16g+15) of entry le
  const int le = t >> 3, g = t & 7;
  const int odd = le & 1;
  const bool godd = (g & 1) != 0;
  const uint32_t psel = odd ? 0x03020706u : 0x05040100u;  // pair (partner, own) high halves / own, partner low
  // paired transposed writes: dword j of this thread goes to row d = 16 g + 2 (j ^ (g & 1)) + odd
  const int slot = tt_slot(le & ~1);
  auto load_tile = [&](int tile, u32x4& v0, u32x4& v1) {
    const uint32_t off = (uint32_t)((e_begin + (int64_t)tile * TE + le) * (TDH * 2) + g * 32);
    v0 = buf_load16(rs, off);
    v1 = buf_load16(rs, off + 16);
  };
  auto stage = [&](int buf, const u32x4& c0, const u32x4& c1) {
    sm.kt[buf][le * 16 + ((2 * g) ^ (le & 15))] = __builtin_bit_cast(uint4, c0);
    sm.kt[buf][le * 16 + ((2 * g + 1) ^ (le & 15))] = __builtin_bit_cast(uint4, c1);
    char* tt = (char*)sm.ktt[buf];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int jj = j ^ (g & 1);
      const u32x4 c = j < 4 ? c0 : c1;
      const uint32_t a0 = c[j & 3], a1 = c[(j ^ 1) & 3];  // compile-time lanes of the vector
      const uint32_t own = godd ? a1 : a0;
      // the partner (entry le ^ 1, same dims, same jj) is lane ^ 8, in the same row of 16 lanes
      const uint32_t part = ror_u<8>(own);
      const uint32_t v = __builtin_amdgcn_perm(part, own, psel);
      const int d = 16 * g + 2 * jj + odd;
      *(uint32_t*)(tt + d * 64 + (((slot >> 3) ^ tt_swz(d)) << 4) + (slot & 7) * 2) = v;
    }
  };
  auto step = [&](int tile, int buf) {
    const int64_t s0 = e_begin + (int64_t)tile * TE;  // first entry of the tile (a multiple of 32)
    __syncthreads();  // the tile is in LDS
    // ---- head dots of 32 entries x this wave's 16 heads
    f32x4 S[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const int e = 16 * mb + hl;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 A = __builtin_bit_cast(bf16x8, sm.kt[buf][e * 16 + ((4 * ks + kg) ^ (e & 15))]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, qh[ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, ql[ks], acc, 0, 0, 0);
      }
      S[mb] = acc;  // S[mb][i]: entry 16mb + 4kg + i, head 16wq + hl
    }
    // ---- partial logits over this wave's heads: sums over the 16 lanes of a row
    float xs[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      float x = wh * fmaxf(S[v >> 2][v & 3], 0.f);
      x += ror<8>(x);
      x += ror<4>(x);
      x += ror<2>(x);
      x += ror<1>(x);
      xs[v] = x;
    }
    if (hl < 8) {  // lane hl writes value hl: entry 16 (hl / 4) + 4 kg + hl % 4
      float x = xs[0];
#pragma unroll
      for (int v = 1; v < 8; ++v) x = hl == v ? xs[v] : x;
      ((float*)&sm.xpart[buf][16 * (hl >> 2) + 4 * kg + (hl & 3)])[wq] = x;
    }
    __syncthreads();
    // ---- loss and g_s = d loss / d x_s: entry e = lane % 32, once per wave (lanes 32..63 repeat it)
    {
      const int e = lane & 31;
      const float4 xp = sm.xpart[buf][e];
      const float x = (xp.x + xp.y) + (xp.z + xp.w);
      const bool valid = s0 + e < n_b;
      const uint32_t lw = (uint32_t)(lab[s0 >> 6] >> (s0 & 63));  // the tile's 32 labels
      float fl, fg;
      focal(x, (lw >> e) & 1, a.gamma, a.alpha, fl, fg);
      const float gv = valid ? fg * a.inv_total : 0.f;
      const uint32_t gp = cvt_bf16x2(gv, gv - __uint_as_float(cvt_bf16x2(gv, 0.f) << 16));
      if (lane < 32) {
        sm.gh[wq][e] = (uint16_t)gp;
        sm.gl[wq][e] = (uint16_t)(gp >> 16);
      }
      if (wq == 0 && lane < 32 && valid) ll += (double)fl;
    }
    __builtin_amdgcn_wave_barrier();  // gh, gl are written and read by this wave only: LDS keeps the wave's order
    // ---- the coefficients g_s [S_sj > 0] as bf16 hi + lo, in registers: lane (head hl, kg) holds
    // entries 16 mb + 4 kg + i, which are slots 8 kg + 4 mb + i. The gate w_j is applied after the
    // scan (dq_j = w_j dq'_j), and dw_j = sum_s g_s ReLU(S_sj) = q_j . dq'_j follows from the same sum.
    u32x4 ch, cl;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const uint2 h2 = *(const uint2*)&sm.gh[wq][16 * mb + 4 * kg];
      const uint2 l2 = *(const uint2*)&sm.gl[wq][16 * mb + 4 * kg];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const uint32_t m = (S[mb][2 * p] > 0.f ? 0x0000FFFFu : 0u) | (S[mb][2 * p + 1] > 0.f ? 0xFFFF0000u : 0u);
        ch[2 * mb + p] = (p ? h2.y : h2.x) & m;
        cl[2 * mb + p] = (p ? l2.y : l2.x) & m;
      }
    }
    const bf16x8 Ah = __builtin_bit_cast(bf16x8, ch), Al = __builtin_bit_cast(bf16x8, cl);
    // ---- dq' for this wave's heads: coefficients (16 heads x 32 slots) x K^T (32 slots x 128 dims)
    const char* tt = (const char*)sm.ktt[buf];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const int d = 16 * nb + hl;
      const bf16x8 Bk = __builtin_bit_cast(bf16x8, *(const uint4*)(tt + d * 64 + ((kg ^ tt_swz(d)) << 4)));
      accb[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ah, Bk, accb[nb], 0, 0, 0);
      accb[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Al, Bk, accb[nb], 0, 0, 0);
    }
  };

  // two tiles in flight; the LDS tiles alternate, so one barrier before the score MFMAs and one
  // before the loss are enough (a wave writes buffer x only after every wave has passed the
  // barriers of the tile that read it last)
  u32x4 ra0, ra1, rb0, rb1;
  load_tile(0, ra0, ra1);
  if (ntiles > 1) load_tile(1, rb0, rb1);
  for (int tile = 0; tile < ntiles; tile += 2) {
    stage(0, ra0, ra1);
    if (tile + 2 < ntiles) load_tile(tile + 2, ra0, ra1);
    step(tile, 0);
    if (tile + 1 < ntiles) {
      stage(1, rb0, rb1);
      if (tile + 3 < ntiles) load_tile(tile + 3, rb0, rb1);
      step(tile + 1, 1);
    }
  }

  // ---- this block's partial sums
  float* part = a.part + (int64_t)blockIdx.x * PW;
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) part[(16 * wq + 4 * kg + i) * TDH + 16 * nb + hl] = accb[nb][i];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ll += __shfl_xor(ll, o);
  if (lane == 0) sm.lsum[wq] = ll;
  __syncthreads();
  if (t == 0) part[TNH * TDH] = (float)(sm.lsum[0] + sm.lsum[1] + sm.lsum[2] + sm.lsum[3]);
}

// dq'[b] = the sum of sequence b's block partials; then dq_j = w_j dq'_j and dw_j = q_j . dq'_j.
// Block (head x, sequence y): 512 threads, thread t sums dim t % 128 of the head over a quarter of the
// blocks (t / 128), the quarters meet in LDS. Block x = TNH of row y = 0 sums the loss.
__global__ __launch_bounds__(512) void train_reduce_kernel(const TrainArgs a) {
  const int b = blockIdx.y;
  const int t = threadIdx.x;
  if (blockIdx.x == TNH) {
    if (b != 0) return;
    __shared__ double red[512];
    double s = 0.0;
    for (int64_t k = t; k < a.nblk; k += 512) s += (double)a.part[k * PW + PW - 1];
    red[t] = s;
    __syncthreads();
    for (int o = 256; o > 0; o >>= 1) {
      if (t < o) red[t] += red[t + o];
      __syncthreads();
    }
    if (t == 0) a.loss[0] = (float)(red[0] * (double)a.inv_total);
    return;
  }
  __shared__ float qs[4][TDH];
  __shared__ float wsum[2];
  const int head = blockIdx.x, dim = t & (TDH - 1), quarter = t >> 7;
  const int j = head * TDH + dim;
  const int64_t be = (int64_t)a.tpb * TE;
  const int64_t k0 = first_block(a.key_off, b, be);
  const int64_t nk = (a.key_off[b + 1] - a.key_off[b] + be - 1) / be;
  const float* p = a.part + j;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int64_t k = k0 + quarter * nk / 4;
  const int64_t k1 = k0 + (quarter + 1) * nk / 4;
  for (; k + 8 <= k1; k += 8)
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] += p[(k + u) * PW];
  for (; k < k1; ++k) acc[0] += p[k * PW];
  qs[quarter][dim] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
  __syncthreads();
  float v = 0.f;
  if (t < TDH) {
    const float s = (qs[0][dim] + qs[1][dim]) + (qs[2][dim] + qs[3][dim]);
    a.dq[(int64_t)b * TNH * TDH + j] = a.w[(int64_t)b * TNH + head] * s;
    v = a.q[(int64_t)b * TNH * TDH + j] * s;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if (t < TDH && (t & 63) == 0) wsum[t >> 6] = v;
  __syncthreads();
  if (t == 0) a.dw[(int64_t)b * TNH + head] = wsum[0] + wsum[1];
}

// Partial dc = dq W^IUQ over a slice of DCR rows o of the w_iuq buffer: dcp[slice][b][k] =
// sum_{o in slice} dq[b][o] W[o][k]. Block: one slice x DCC columns; wave w takes rows o = w, w+4, ...
// of the slice, lane l columns 4l..4l+3, with 16 rows' loads in flight at a time; the four waves' sums
// meet in LDS.
constexpr int DCR = TNH * TDH / kTrainDcSlices;
constexpr int DCC = 256;
__global__ __launch_bounds__(256) void train_dc_kernel(const TrainArgs a) {
  __shared__ float dqs[DCR][33];
  __shared__ float4 red[3][8][DCC / 4];
  const int t = threadIdx.x, wv = t >> 6, lane = t & 63;
  const int o0 = blockIdx.x * DCR;
  const int k = blockIdx.y * DCC + lane * 4;
  for (int i = t; i < DCR * a.B; i += 256) dqs[i % DCR][i / DCR] = a.dq[(int64_t)(i / DCR) * TNH * TDH + o0 + i % DCR];
  __syncthreads();
  const bool col_ok = k < a.r;
  const uint16_t* W = (const uint16_t*)a.w_iuq;
  for (int b0 = 0; b0 < a.B; b0 += 8) {
    float acc[8][4];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[u][c] = 0.f;
    if (col_ok) {
      constexpr int RU = 16;  // rows of this wave with loads in flight together
      for (int o1 = wv; o1 < DCR; o1 += 4 * RU) {
        uint2 raw[RU];
#pragma unroll
        for (int u = 0; u < RU; ++u) raw[u] = *(const uint2*)(W + (int64_t)(o0 + o1 + 4 * u) * a.r + k);
#pragma unroll
        for (int ru = 0; ru < RU; ++ru) {
          const int o = o1 + 4 * ru;
          const float w4[4] = {bf16_bits_to_f32(raw[ru].x & 0xFFFFu), bf16_bits_to_f32(raw[ru].x >> 16),
                               bf16_bits_to_f32(raw[ru].y & 0xFFFFu), bf16_bits_to_f32(raw[ru].y >> 16)};
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const float dv = b0 + u < a.B ? dqs[o][b0 + u] : 0.f;
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[u][c] = fmaf(dv, w4[c], acc[u][c]);
          }
        }
      }
    }
    if (wv > 0)
#pragma unroll
      for (int u = 0; u < 8; ++u) red[wv - 1][u][lane] = make_float4(acc[u][0], acc[u][1], acc[u][2], acc[u][3]);
    __syncthreads();
    if (wv == 0 && col_ok)
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (b0 + u >= a.B) break;
        float4 o4 = make_float4(acc[u][0], acc[u][1], acc[u][2], acc[u][3]);
#pragma unroll
        for (int w2 = 0; w2 < 3; ++w2) {
          const float4 x = red[w2][u][lane];
          o4.x += x.x; o4.y += x.y; o4.z += x.z; o4.w += x.w;
        }
        *(float4*)(a.dcp + ((int64_t)blockIdx.x * a.B + b0 + u) * a.r + k) = o4;
      }
    __syncthreads();  // red is reused by the next group of 8 sequences
  }
}

// out[i] = sum over p < nparts of in[p * n + i]
__global__ __launch_bounds__(256) void train_sum_kernel(const float* __restrict__ in, int nparts, int64_t n,
                                                      float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float acc[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) acc[u] = 0.f;
  int p = 0;
  for (; p + 16 <= nparts; p += 16)
#pragma unroll
    for (int u = 0; u < 16; ++u) acc[u] += in[(int64_t)(p + u) * n + i];
  for (; p < nparts; ++p) acc[0] += in[(int64_t)p * n + i];
#pragma unroll
  for (int w = 8; w > 0; w >>= 1)
#pragma unroll
    for (int u = 0; u < w; ++u) acc[u] += acc[u + w];
  out[i] = acc[0];
}

// out[i][j] = sum_b u[b][i] v[b][j] (u fp32 with row stride I, v fp32 or bf16 with row stride J, J a
// multiple of 4). Block: 16 rows i x 1024 columns j, four consecutive columns per thread (16-byte stores).
// One launch can hold two such products: blocks y < ny0 form the first (u, I, out), the others the
// second (u1, I1, out1), over the same v.
template <bool VBF16>
__global__ __launch_bounds__(256) void train_outer_kernel(const float* __restrict__ u, const void* __restrict__ v,
                                                        int B, int64_t I, int64_t J, float* __restrict__ out,
                                                        int ny0, const float* __restrict__ u1, int64_t I1,
                                                        float* __restrict__ out1) {
  __shared__ float4 us[32][4];  // [b][i / 4]
  int by = blockIdx.y;
  if (by >= ny0) {
    by -= ny0;
    u = u1;
    I = I1;
    out = out1;
  }
  const int64_t i0 = (int64_t)by * 16;
  const int64_t j = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  for (int x = threadIdx.x; x < 16 * B; x += 256) {
    const int bb = x / 16, ii = x % 16;
    ((float*)us[bb])[ii] = i0 + ii < I ? u[(int64_t)bb * I + i0 + ii] : 0.f;
  }
  __syncthreads();
  if (j >= J) return;
  float s[16][4];
#pragma unroll
  for (int ii = 0; ii < 16; ++ii)
#pragma unroll
    for (int c = 0; c < 4; ++c) s[ii][c] = 0.f;
  for (int bb = 0; bb < B; ++bb) {
    float x[4];
    if constexpr (VBF16) {
      const uint2 raw = *(const uint2*)((const uint16_t*)v + (int64_t)bb * J + j);
      x[0] = bf16_bits_to_f32(raw.x & 0xFFFFu);
      x[1] = bf16_bits_to_f32(raw.x >> 16);
      x[2] = bf16_bits_to_f32(raw.y & 0xFFFFu);
      x[3] = bf16_bits_to_f32(raw.y >> 16);
    } else {
      const float4 f = *(const float4*)((const float*)v + (int64_t)bb * J + j);
      x[0] = f.x; x[1] = f.y; x[2] = f.z; x[3] = f.w;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 cu = us[bb][q];
      const float cv[4] = {cu.x, cu.y, cu.z, cu.w};
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) s[4 * q + r][c] = fmaf(cv[r], x[c], s[4 * q + r][c]);
    }
  }
  const int nrow = (int)min((int64_t)16, I - i0);
#pragma unroll
  for (int ii = 0; ii < 16; ++ii)
    if (ii < nrow) *(float4*)(out + (i0 + ii) * J + j) = make_float4(s[ii][0], s[ii][1], s[ii][2], s[ii][3]);
}

__global__ __launch_bounds__(256) void train_zero_kernel(float* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

}  // namespace

hipError_t launch_train_zero(float* p, int64_t n, hipStream_t st) {
  if (n > 0) hipLaunchKernelGGL(train_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

int64_t train_scan_blocks(const int64_t* key_off_host, int B, int* tpb_out) {
  int64_t tiles = 0;
  for (int b = 0; b < B; ++b) tiles += (key_off_host[b + 1] - key_off_host[b] + TE - 1) / TE;
  const int64_t tpb = std::max<int64_t>(MIN_TPB, (tiles + SCAN_BLOCKS - 1) / SCAN_BLOCKS);
  int64_t s = 0;
  for (int b = 0; b < B; ++b) s += (key_off_host[b + 1] - key_off_host[b] + tpb * TE - 1) / (tpb * TE);
  if (tpb_out) *tpb_out = (int)tpb;
  return s;
}

// Workspace: c [B][r], q [B][n_h d_h], w [B][n_h], dq, dw, dc, the dc partials, then the scan
// blocks' partials (PW floats each, odd, so they come last).
TrainWs train_carve(void* ws, int B, int r, int64_t nblk) {
  TrainWs o{};
  size_t off = 0;  // in floats
  auto take = [&](float*& p, int64_t n) {
    p = ws ? (float*)ws + off : nullptr;
    off += (size_t)n;
  };
  take(o.c, (int64_t)B * r);
  take(o.q, (int64_t)B * TNH * TDH);
  take(o.w, (int64_t)B * TNH);
  take(o.dq, (int64_t)B * TNH * TDH);
  take(o.dw, (int64_t)B * TNH);
  take(o.dc, (int64_t)B * r);
  take(o.dcp, (int64_t)kTrainDcSlices * B * r);
  take(o.part, nblk * PW);
  o.bytes = off * sizeof(float);
  return o;
}

size_t train_workspace_bytes(int B, int r, int64_t nblk) { return train_carve(nullptr, B, r, nblk).bytes + 256; }

hipError_t launch_train(const TrainArgs& a, hipStream_t st) {
  hipError_t e;
  if (a.nblk > 0) {
    hipLaunchKernelGGL(train_scan_kernel, dim3((unsigned)a.nblk), dim3(TT), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(train_reduce_kernel, dim3(TNH + 1, a.B), dim3(512), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int nrb = TNH * TDH / DCR;
  hipLaunchKernelGGL(train_dc_kernel, dim3(nrb, (a.r + DCC - 1) / DCC), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t ndc = (int64_t)a.B * a.r;
  hipLaunchKernelGGL(train_sum_kernel, dim3((unsigned)((ndc + 255) / 256)), dim3(256), 0, st, a.dcp, nrb, ndc, a.dc);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // g_iuq = dq^T c; then g_dq = dc^T h and g_w = dw^T h in one launch
  const int ny_iuq = (TNH * TDH + 15) / 16;
  hipLaunchKernelGGL(train_outer_kernel<false>, dim3((a.r + 1023) / 1024, ny_iuq), dim3(256), 0, st, a.dq,
                     (const void*)a.c, a.B, (int64_t)TNH * TDH, (int64_t)a.r, a.g_iuq, ny_iuq, (const float*)nullptr,
                     (int64_t)0, (float*)nullptr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int ny_dq = (a.r + 15) / 16, ny_w = (TNH + 15) / 16;
  hipLaunchKernelGGL(train_outer_kernel<true>, dim3((a.d + 1023) / 1024, ny_dq + ny_w), dim3(256), 0, st, a.dc, a.h,
                     a.B, (int64_t)a.r, (int64_t)a.d, a.g_dq, ny_dq, (const float*)a.dw, (int64_t)TNH, a.g_w);
  return hipGetLastError();
}

}  // namespace lsa
