// Indexer query projection ([BLOG] §3.1 of the FlashMemory-DeepSeek-V4
// write-up): c = h W^DQ (rank r), q = c W^IUQ, w = h W^w.
//
// These are GEMMs with a tiny M (the batch of sequences, B <= 128) and large
// weights. Their cost is streaming the weights from HBM once. The weights use
// the "out x in" layout, so each output row's weights are contiguous along the
// reduction dimension. They serve as the MFMA A operand (16 output rows per
// block) and the batch is the B operand (16 columns per MFMA). A block of four
// waves splits the reduction four ways and sums the partials through LDS.
//   stage 1 (down): rows = r outputs of c plus n_h gate outputs, K = d, B operand = h
//   stage 2 (up):   rows = n_h*d_h outputs of q,                  K = r, B operand = c
// bf16 weights use v_mfma_f32_16x16x32_bf16. In stage 2 the fp32 latent c is
// split into bf16 hi + lo as two column halves of the same MFMA (columns 0..7
// hi, 8..15 lo for 8 sequences), and the halves are added with one lane swap.
// fp32 weights use v_mfma_f32_16x16x4f32.
//
// 16x16 MFMA layout (wave64): A lane l -> row l%16, k-group l/16;
// B lane l -> column l%16, k-group l/16; D lane l -> rows 4*(l/16)+i, column l%16.
#include "kernels.hpp"

namespace lsa {

static constexpr int PJ_THREADS = 256;

template <bool F32, bool UP, int NB>
__global__ __launch_bounds__(PJ_THREADS) void project_kernel(const ProjArgs a) {
  constexpr int KCH = F32 ? 4 : 32;            // k per MFMA
  constexpr int COLS = (UP && !F32) ? 8 : 16;  // sequences per column block
  __shared__ f32x4 red[3][NB][64];

  const int l = blockIdx.y;
  const int lane = threadIdx.x & 63, m = lane & 15, kg = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int K = UP ? a.r : a.d;
  const int rows = UP ? a.n_h * a.d_h : a.r + a.n_h;
  const int rb = blockIdx.x * 16;

  // A operand row of this lane
  const int R = rb + m;
  const char* arow = nullptr;
  const int esz = F32 ? 4 : 2;
  if (UP) {
    if (R < rows) arow = (const char*)a.w_iuq[l] + (int64_t)R * K * esz;
  } else {
    if (R < a.r) arow = (const char*)a.w_dq[l] + (int64_t)R * K * esz;
    else if (R < rows) arow = (const char*)a.w_w[l] + (int64_t)(R - a.r) * K * esz;
  }

  f32x4 acc[NB];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) acc[cb] = f32x4{0, 0, 0, 0};

  const int chunks = K / KCH;
  const int c0 = wv * chunks / 4, c1 = (wv + 1) * chunks / 4;
  for (int c = c0; c < c1; ++c) {
    const int k0 = c * KCH + (F32 ? kg : 8 * kg);
    if constexpr (F32) {
      const float av = arow ? ((const float*)arow)[k0] : 0.0f;
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        const int seq = cb * COLS + m;
        float bv = 0.0f;
        if (seq < a.B) {
          bv = UP ? a.c[l][(int64_t)seq * a.r + k0] : ((const float*)a.h[l])[(int64_t)seq * a.d + k0];
        }
        acc[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[cb], 0, 0, 0);
      }
    } else {
      const bf16x8 av = as_bf16x8(arow ? *(const u32x4*)(arow + (int64_t)k0 * 2) : u32x4{0, 0, 0, 0});
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        bf16x8 bv;
        if constexpr (UP) {
          const int seq = cb * COLS + (m & 7);
          if (seq < a.B) {
            const float* cp = a.c[l] + (int64_t)seq * a.r + k0;
            const f32x4 v0 = *(const f32x4*)cp, v1 = *(const f32x4*)(cp + 4);
            float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
            bf16x8 hi, lo;
            split8(v, hi, lo);
            bv = (m & 8) ? lo : hi;
          } else {
            bv = as_bf16x8(u32x4{0, 0, 0, 0});
          }
        } else {
          const int seq = cb * COLS + m;
          bv = as_bf16x8(seq < a.B ? *(const u32x4*)((const char*)a.h[l] + ((int64_t)seq * a.d + k0) * 2)
                                   : u32x4{0, 0, 0, 0});
        }
        acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[cb], 0, 0, 0);
      }
    }
  }

  // sum the four waves' partial products
  if (wv > 0) {
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) red[wv - 1][cb][lane] = acc[cb];
  }
  __syncthreads();
  if (wv != 0) return;
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    f32x4 s = acc[cb];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const f32x4 t = red[j][cb][lane];
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
      const int row = rb + 4 * kg + i;
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

template <bool F32, bool UP>
static hipError_t launch_stage(const ProjArgs& a, int L, int nb, hipStream_t st) {
  const int rows = UP ? a.n_h * a.d_h : a.r + a.n_h;
  const dim3 grid((rows + 15) / 16, L);
#define LSA_PJ(NB_) hipLaunchKernelGGL((project_kernel<F32, UP, NB_>), grid, dim3(PJ_THREADS), 0, st, a)
  if (nb <= 1) LSA_PJ(1);
  else if (nb <= 2) LSA_PJ(2);
  else if (nb <= 4) LSA_PJ(4);
  else if (nb <= 8) LSA_PJ(8);
  else LSA_PJ(16);  // B <= 128: at most 16 column blocks
#undef LSA_PJ
  return hipGetLastError();
}

hipError_t launch_project(const ProjArgs& a, int L, bool f32, hipStream_t st) {
  hipError_t e;
  if (f32) {
    const int nb = (a.B + 15) / 16;
    if ((e = launch_stage<true, false>(a, L, nb, st)) != hipSuccess) return e;
    return launch_stage<true, true>(a, L, nb, st);
  }
  if ((e = launch_stage<false, false>(a, L, (a.B + 15) / 16, st)) != hipSuccess) return e;
  return launch_stage<false, true>(a, L, (a.B + 7) / 8, st);
}

}  // namespace lsa
