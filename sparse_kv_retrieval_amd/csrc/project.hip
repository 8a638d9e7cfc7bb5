// Indexer query projection ([BLOG] §3.1 of the FlashMemory-DeepSeek-V4
// write-up): c = h W^DQ (rank r), q = c W^IUQ, w = h W^w.
//
// Two forms. project_kernel reads the weights in their plain "out x in"
// layout (lsa_project). project_packed_kernel reads weights rearranged once
// into the MFMA operand layout (lsa_pack_weights, lsa_project_packed), so each
// weight load is one contiguous 1 KiB wave access; it is the faster form for
// bf16. The notes below describe the plain form.
//
// These are GEMMs with a tiny M (the batch of sequences, B <= 128) and large
// weights. Their cost is streaming the weights from HBM once. The weights use
// the "out x in" layout, so each output row's weights are contiguous along the
// reduction dimension. They serve as the MFMA A operand and the batch is the
// B operand (16 columns per MFMA). A block covers 16*MB output rows. Its four
// waves split the reduction four ways and sum the partials through LDS. The
// reduction loop is unrolled KU chunks deep, with all loads issued first, so
// each wave keeps several KiB of weights in flight.
//   stage 1 (down): rows = r outputs of c plus n_h gate outputs, K = d, B operand = h
//   stage 2 (up):   rows = n_h*d_h outputs of q,                  K = r, B operand = c
// bf16 weights use v_mfma_f32_16x16x32_bf16. In stage 2 the fp32 latent c is
// split into bf16 hi + lo as two column halves of the same MFMA (columns 0..7
// hi, 8..15 lo for 8 sequences), and the halves are added with one lane swap.
// Each split is reused for the block's MB row groups. fp32 weights use
// v_mfma_f32_16x16x4f32.
//
// 16x16 MFMA layout (wave64): A lane l -> row l%16, k-group l/16;
// B lane l -> column l%16, k-group l/16; D lane l -> rows 4*(l/16)+i, column l%16.
#include "kernels.hpp"

namespace lsa {

static constexpr int PJ_THREADS = 256;

template <bool F32, bool UP, int NB, int MB>
__global__ __launch_bounds__(PJ_THREADS) void project_kernel(const ProjArgs a) {
  constexpr int KCH = F32 ? 4 : 32;            // k per MFMA
  constexpr int COLS = (UP && !F32) ? 8 : 16;  // sequences per column block
  constexpr int KU = F32 ? 8 : 4;              // reduction chunks per unrolled step
  __shared__ f32x4 red[3][MB][NB][64];

  const int l = blockIdx.y;
  const int lane = threadIdx.x & 63, m = lane & 15, kg = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int K = UP ? a.r : a.d;
  const int rows = UP ? a.n_h * a.d_h : a.r + a.n_h;
  const int rb = blockIdx.x * 16 * MB;
  const int esz = F32 ? 4 : 2;

  // A operand rows of this lane (one per row group)
  const char* arow[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int R = rb + 16 * mb + m;
    arow[mb] = nullptr;
    if (UP) {
      if (R < rows) arow[mb] = (const char*)a.w_iuq[l] + (int64_t)R * K * esz;
    } else {
      if (R < a.r) arow[mb] = (const char*)a.w_dq[l] + (int64_t)R * K * esz;
      else if (R < rows) arow[mb] = (const char*)a.w_w[l] + (int64_t)(R - a.r) * K * esz;
    }
  }

  f32x4 acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) acc[mb][cb] = f32x4{0, 0, 0, 0};

  // the reduction is split over the block's four waves and over gridDim.z blocks; with more than one
  // block per output (gridDim.z == 2), both add into outputs the caller has zeroed, and 0 + a + b
  // rounds the same in either order
  const int ks = gridDim.z;
  const int chunks = K / KCH;
  const int part = (int)blockIdx.z * 4 + wv;
  const int c0 = part * chunks / (4 * ks), c1 = (part + 1) * chunks / (4 * ks);

  // one reduction chunk: k0 is this lane's first k
  auto b_frag_bf16 = [&](int cb, int k0) -> bf16x8 {
    if constexpr (UP) {
      const int seq = cb * COLS + (m & 7);
      if (seq >= a.B) return as_bf16x8(u32x4{0, 0, 0, 0});
      const float* cp = a.c[l] + (int64_t)seq * a.r + k0;
      const f32x4 v0 = *(const f32x4*)cp, v1 = *(const f32x4*)(cp + 4);
      float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      bf16x8 hi, lo;
      split8(v, hi, lo);
      return (m & 8) ? lo : hi;
    } else {
      const int seq = cb * COLS + m;
      return as_bf16x8(seq < a.B ? *(const u32x4*)((const char*)a.h[l] + ((int64_t)seq * a.d + k0) * 2)
                                 : u32x4{0, 0, 0, 0});
    }
  };
  auto b_frag_f32 = [&](int cb, int k0) -> float {
    const int seq = cb * COLS + m;
    if (seq >= a.B) return 0.0f;
    return UP ? a.c[l][(int64_t)seq * a.r + k0] : ((const float*)a.h[l])[(int64_t)seq * a.d + k0];
  };

  int c = c0;
  for (; c + KU <= c1; c += KU) {
    if constexpr (F32) {
      float av[KU][MB], bv[KU][NB];
#pragma unroll
      for (int u = 0; u < KU; ++u) {
        const int k0 = (c + u) * KCH + kg;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) av[u][mb] = arow[mb] ? ((const float*)arow[mb])[k0] : 0.0f;
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) bv[u][cb] = b_frag_f32(cb, k0);
      }
#pragma unroll
      for (int u = 0; u < KU; ++u)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int cb = 0; cb < NB; ++cb)
            acc[mb][cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u][mb], bv[u][cb], acc[mb][cb], 0, 0, 0);
    } else {
      bf16x8 av[KU][MB], bv[KU][NB];
#pragma unroll
      for (int u = 0; u < KU; ++u) {
        const int k0 = (c + u) * KCH + 8 * kg;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          av[u][mb] = as_bf16x8(arow[mb] ? __builtin_nontemporal_load((const u32x4*)(arow[mb] + (int64_t)k0 * 2))
                                         : u32x4{0, 0, 0, 0});
      }
#pragma unroll
      for (int u = 0; u < KU; ++u)
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) bv[u][cb] = b_frag_bf16(cb, (c + u) * KCH + 8 * kg);
#pragma unroll
      for (int u = 0; u < KU; ++u)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int cb = 0; cb < NB; ++cb)
            acc[mb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[u][mb], bv[u][cb], acc[mb][cb], 0, 0, 0);
    }
  }
  for (; c < c1; ++c) {
    if constexpr (F32) {
      const int k0 = c * KCH + kg;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const float av = arow[mb] ? ((const float*)arow[mb])[k0] : 0.0f;
#pragma unroll
        for (int cb = 0; cb < NB; ++cb)
          acc[mb][cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, b_frag_f32(cb, k0), acc[mb][cb], 0, 0, 0);
      }
    } else {
      const int k0 = c * KCH + 8 * kg;
      bf16x8 bv[NB];
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) bv[cb] = b_frag_bf16(cb, k0);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const bf16x8 av = as_bf16x8(arow[mb] ? *(const u32x4*)(arow[mb] + (int64_t)k0 * 2) : u32x4{0, 0, 0, 0});
#pragma unroll
        for (int cb = 0; cb < NB; ++cb)
          acc[mb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv[cb], acc[mb][cb], 0, 0, 0);
      }
    }
  }

  // sum the four waves' partial products
  if (wv > 0) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) red[wv - 1][mb][cb][lane] = acc[mb][cb];
  }
  __syncthreads();
  if (wv != 0) return;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      f32x4 s = acc[mb][cb];
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const f32x4 t = red[j][mb][cb][lane];
        s[0] += t[0]; s[1] += t[1]; s[2] += t[2]; s[3] += t[3];
      }
      if constexpr (UP && !F32) {
        // column m holds the hi part (m < 8) or the lo part (m >= 8) of sequence cb*8 + (m&7)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[i] += __shfl_xor(s[i], 8);
        if (m & 8) continue;
      }
      const int seq = cb * COLS + (UP && !F32 ? (m & 7) : m);
      if (seq >= a.B) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = rb + 16 * mb + 4 * kg + i;
        if (row >= rows) continue;
        float* dst = UP ? &a.q[l][(int64_t)seq * rows + row]
                        : row < a.r ? &a.c[l][(int64_t)seq * a.r + row] : &a.w[l][(int64_t)seq * a.n_h + (row - a.r)];
        if (ks > 1)
          unsafeAtomicAdd(dst, s[i]);
        else
          *dst = s[i];
      }
    }
  }
}

// bf16 weights in the packed operand layout (lsa_pack_weights). A matrix of
// `rows` x K (out x in) is stored as ceil(rows/16) x (K/32) blocks of 1 KiB.
// Block (rb, ch) holds rows 16rb..16rb+15 and columns 32ch..32ch+31 in lane
// order: lane l = 16kg + m owns the 16 bytes of row 16rb+m, columns
// 32ch+8kg..32ch+8kg+7, which is exactly its A operand of the 16x16x32 MFMA.
// Rows past the end are zero. Every weight load is then one contiguous 1 KiB
// wave access, and a wave walking along K streams contiguous memory.
//
// W waves per block split the reduction. Each wave streams its slice of K in
// batches of KU chunks, double-buffered: batch i+1's loads are in flight while
// batch i's MFMAs run. Every load is a raw buffer load issued on every path:
// row groups past the end, sequences past B and chunks past the wave's slice
// read out of range as zeros, which add nothing to the MFMA sums. A block's
// rows lie in one weight matrix (W^DQ or W^w), so its buffer resource is
// uniform. The W partial sums are added through LDS in wave order, so the
// result does not depend on timing.
template <bool UP, int MB, int NB, int W, int KU>
__global__ __launch_bounds__(64 * W) void project_packed_kernel(const ProjArgs a) {
  constexpr int KCH = 32;                 // k per MFMA
  constexpr int COLS = UP ? 8 : 16;       // sequences per column block (UP: 8 hi + 8 lo columns)
  constexpr int BV = UP ? 2 : 1;          // 16-byte B loads per chunk (UP: 8 fp32 of c)
  __shared__ f32x4 red[W - 1][MB][NB][64];

  const int l = blockIdx.y;
  const int lane = threadIdx.x & 63, m = lane & 15, kg = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int K = UP ? a.r : a.d;
  const int rows = UP ? a.n_h * a.d_h : a.r + a.n_h;
  const int rb = blockIdx.x * 16 * MB;

  // packed weight matrix of this block, and this lane's offsets in it
  const bool gate_rows = !UP && rb >= a.r;
  const char* wbase = UP ? (const char*)a.w_iuq[l] : gate_rows ? (const char*)a.w_w[l] : (const char*)a.w_dq[l];
  const int r0 = gate_rows ? a.r : 0;
  const int nrb = ((UP ? rows : gate_rows ? a.n_h : a.r) + 15) / 16;  // 16-row blocks of the matrix
  const int chunks = K / KCH;
  const auto ra = buf_rsrc(wbase, (uint32_t)nrb * chunks * 1024);
  uint32_t aoff[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int rbk = (rb - r0) / 16 + mb;
    aoff[mb] = rbk < nrb ? (uint32_t)rbk * chunks * 1024 + 16 * lane : BUF_OOB;
  }
  // B operand: h (bf16) or c (fp32), one row per sequence
  const auto rbuf = UP ? buf_rsrc(a.c[l], (uint32_t)a.B * a.r * 4) : buf_rsrc(a.h[l], (uint32_t)a.B * a.d * 2);
  uint32_t boff[NB];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    const int seq = cb * COLS + (UP ? (m & 7) : m);
    boff[cb] = seq < a.B ? (UP ? (uint32_t)seq * a.r * 4 + 32 * kg : (uint32_t)seq * a.d * 2 + 16 * kg) : BUF_OOB;
  }

  const int c0 = wv * chunks / W, c1 = (wv + 1) * chunks / W;
  const int nbat = (c1 - c0 + KU - 1) / KU;

  u32x4 A0[KU][MB], A1[KU][MB], B0[KU][NB][BV], B1[KU][NB][BV];
  f32x4 acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) acc[mb][cb] = f32x4{0, 0, 0, 0};

#define LSA_PJ_LOAD(AA, BB, BAT)                                                                    \
  do {                                                                                            \
    _Pragma("unroll") for (int u = 0; u < KU; ++u) {                                              \
      const int ch = c0 + (BAT) * KU + u;                                                         \
      const bool ok = ch < c1;                                                                    \
      _Pragma("unroll") for (int mb = 0; mb < MB; ++mb)                                           \
        AA[u][mb] = buf_load16_nt(ra, ok && aoff[mb] != BUF_OOB ? aoff[mb] + ch * 1024 : BUF_OOB);    \
      _Pragma("unroll") for (int cb = 0; cb < NB; ++cb)                                           \
        _Pragma("unroll") for (int v = 0; v < BV; ++v)                                            \
          BB[u][cb][v] = buf_load16(rbuf, ok && boff[cb] != BUF_OOB                               \
                                              ? boff[cb] + ch * KCH * (UP ? 4 : 2) + 16 * v : BUF_OOB); \
    }                                                                                             \
  } while (0)
#define LSA_PJ_MMA(AA, BB)                                                                        \
  do {                                                                                            \
    _Pragma("unroll") for (int u = 0; u < KU; ++u) {                                              \
      bf16x8 bv[NB];                                                                              \
      _Pragma("unroll") for (int cb = 0; cb < NB; ++cb) {                                         \
        if constexpr (UP) {                                                                       \
          float v8[8];                                                                            \
          _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                         \
            v8[i] = __uint_as_float(BB[u][cb][0][i]);                                             \
            v8[4 + i] = __uint_as_float(BB[u][cb][BV - 1][i]);                                    \
          }                                                                                       \
          bf16x8 hi, lo;                                                                          \
          split8(v8, hi, lo);                                                                     \
          bv[cb] = (m & 8) ? lo : hi;                                                             \
        } else {                                                                                  \
          bv[cb] = as_bf16x8(BB[u][cb][0]);                                                       \
        }                                                                                         \
      }                                                                                           \
      _Pragma("unroll") for (int mb = 0; mb < MB; ++mb)                                           \
        _Pragma("unroll") for (int cb = 0; cb < NB; ++cb)                                         \
          acc[mb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(AA[u][mb]), bv[cb], acc[mb][cb], 0, 0, 0); \
    }                                                                                             \
  } while (0)

  LSA_PJ_LOAD(A0, B0, 0);
  for (int bat = 0; bat < nbat; bat += 2) {
    LSA_PJ_LOAD(A1, B1, bat + 1);
    LSA_PJ_MMA(A0, B0);
    LSA_PJ_LOAD(A0, B0, bat + 2);
    LSA_PJ_MMA(A1, B1);
  }
#undef LSA_PJ_LOAD
#undef LSA_PJ_MMA

  // sum the W waves' partial products in wave order
  if (wv > 0) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) red[wv - 1][mb][cb][lane] = acc[mb][cb];
  }
  __syncthreads();
  if (wv != 0) return;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      f32x4 s = acc[mb][cb];
#pragma unroll
      for (int j = 0; j < W - 1; ++j) {
        const f32x4 t = red[j][mb][cb][lane];
        s[0] += t[0]; s[1] += t[1]; s[2] += t[2]; s[3] += t[3];
      }
      if constexpr (UP) {
        // column m holds the hi part (m < 8) or the lo part (m >= 8) of sequence cb*8 + (m&7)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[i] += __shfl_xor(s[i], 8);
        if (m & 8) continue;
      }
      const int seq = cb * COLS + (UP ? (m & 7) : m);
      if (seq >= a.B) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = rb + 16 * mb + 4 * kg + i;
        if (row >= rows) continue;
        if (UP) {
          a.q[l][(int64_t)seq * rows + row] = s[i];
        } else if (row < a.r) {
          a.c[l][(int64_t)seq * a.r + row] = s[i];
        } else {
          a.w[l][(int64_t)seq * a.n_h + (row - a.r)] = s[i];
        }
      }
    }
  }
}

template <bool F32, bool UP, int MB, int NBMAX>
static hipError_t launch_stage(const ProjArgs& a, int L, int nb, hipStream_t st, int ks = 1) {
  const int rows = UP ? a.n_h * a.d_h : a.r + a.n_h;
  const dim3 grid((rows + 16 * MB - 1) / (16 * MB), L, ks);
#define LSA_PJ(NB_) hipLaunchKernelGGL((project_kernel<F32, UP, NB_, MB>), grid, dim3(PJ_THREADS), 0, st, a)
  if (nb <= 1) LSA_PJ(1);
  else if (nb <= 2) LSA_PJ(2);
  else if (nb <= 4 || NBMAX <= 4) LSA_PJ((NBMAX < 4 ? NBMAX : 4));
  else if (nb <= 8) LSA_PJ((NBMAX < 8 ? NBMAX : 8));
  else LSA_PJ(NBMAX);  // B <= 128: at most 16 column blocks
#undef LSA_PJ
  return hipGetLastError();
}

// Rearrange a bf16 "out x in" matrix into the packed operand layout: one
// thread per 16-byte unit of the output.
__global__ __launch_bounds__(256) void pack_weights_kernel(const uint16_t* __restrict__ w, int rows, int K,
                                                           u32x4* __restrict__ out, int64_t units) {
  const int chunks = K / 32;
  for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < units; u += (int64_t)gridDim.x * 256) {
    const int64_t rbk = u / (chunks * 64);
    const int rem = (int)(u - rbk * chunks * 64);
    const int ch = rem / 64, lane = rem % 64;
    const int64_t R = rbk * 16 + (lane & 15);
    const int k0 = ch * 32 + 8 * (lane >> 4);
    out[u] = R < rows ? *(const u32x4*)(w + R * K + k0) : u32x4{0, 0, 0, 0};
  }
}

hipError_t launch_pack_weights(const void* w, int rows, int K, void* out, hipStream_t st) {
  const int64_t units = (int64_t)((rows + 15) / 16) * (K / 32) * 64;
  const int grid = (int)std::min<int64_t>((units + 255) / 256, 65536);
  hipLaunchKernelGGL(pack_weights_kernel, dim3(grid), dim3(256), 0, st, (const uint16_t*)w, rows, K, (u32x4*)out,
                     units);
  return hipGetLastError();
}

template <bool UP, int MB, int NB, int W, int KU>
static hipError_t launch_bf16(const ProjArgs& a, int L, hipStream_t st) {
  const int rows = UP ? a.n_h * a.d_h : a.r + a.n_h;
  const dim3 grid((rows + 16 * MB - 1) / (16 * MB), L);
  hipLaunchKernelGGL((project_packed_kernel<UP, MB, NB, W, KU>), grid, dim3(64 * W), 0, st, a);
  return hipGetLastError();
}

// Block shapes of the packed projection, per stage and number of column blocks NB
// (measured on MI355X at B = 8 and B = 32): MB row groups of 16 rows, W waves
// splitting K, KU chunks per load batch.
template <bool UP>
static hipError_t launch_packed_stage(const ProjArgs& a, int L, int nb, hipStream_t st) {
  if constexpr (UP) {
    if (nb <= 1) return launch_bf16<true, 2, 1, 4, 4>(a, L, st);
    if (nb <= 2) return launch_bf16<true, 4, 2, 4, 2>(a, L, st);
    return launch_bf16<true, 4, 4, 4, 2>(a, L, st);
  } else {
    if (nb <= 1) return launch_bf16<false, 1, 1, 4, 4>(a, L, st);
    return launch_bf16<false, 2, 2, 8, 4>(a, L, st);
  }
}

hipError_t launch_project_packed(const ProjArgs& a, int L, hipStream_t st) {
  hipError_t e;
  const int nb_down = (a.B + 15) / 16, nb_up = (a.B + 7) / 8;
  if ((e = launch_packed_stage<false>(a, L, nb_down, st)) != hipSuccess) return e;
  return launch_packed_stage<true>(a, L, nb_up, st);
}

hipError_t launch_project(const ProjArgs& a, int L, bool f32, hipStream_t st) {
  hipError_t e;
  const int nb_down = (a.B + 15) / 16, nb_up = (a.B + 7) / 8;
  if (f32) {
    const int nb = (a.B + 15) / 16;
    if ((e = launch_stage<true, false, 1, 16>(a, L, nb, st)) != hipSuccess) return e;
    return launch_stage<true, true, 1, 16>(a, L, nb, st);
  }
  if ((e = launch_stage<false, false, 1, 16>(a, L, nb_down, st)) != hipSuccess) return e;
  // the up stage reuses each hi/lo split of c across 4 row groups while the B operand stays small
  if (nb_up <= 4) return launch_stage<false, true, 4, 4>(a, L, nb_up, st);
  return launch_stage<false, true, 1, 16>(a, L, nb_up, st);
}

hipError_t launch_project_split2(const ProjArgs& a, hipStream_t st) {
  hipError_t e;
  const int nb_down = (a.B + 15) / 16, nb_up = (a.B + 7) / 8;
  if ((e = launch_stage<false, false, 1, 16>(a, 1, nb_down, st, 2)) != hipSuccess) return e;
  if (nb_up <= 4) return launch_stage<false, true, 4, 4>(a, 1, nb_up, st, 2);
  return launch_stage<false, true, 1, 16>(a, 1, nb_up, st, 2);
}

}  // namespace lsa
