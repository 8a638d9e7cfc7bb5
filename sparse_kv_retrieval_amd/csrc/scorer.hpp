// MFMA micro-kernel for the head-gated ReLU score of 32 entries by one wave.
//
//   x_s = sum_j w_j * ReLU(q_j . K_s)
//
// This is the lookahead index score before its sigmoid ([BLOG] §3.1 of the
// FlashMemory-DeepSeek-V4 write-up) and also the native Lightning-Indexer
// score ([BLOG] §2.2). The contraction q_j . K_s is a [heads x d_h] x
// [d_h x 32 entries] matrix product on the matrix cores. Heads are the MFMA
// rows, so each lane ends up holding one entry's dot products for 16 heads per
// 32-head block, and the gate/ReLU/head-sum epilogue needs one cross-lane add.
//
// Operand layout (wave64, 32x32 MFMA, one block):
//   A (query):  lane l supplies row (l % 32), k-group (l / 32)
//   B (keys):   lane l supplies column (l % 32), k-group (l / 32)
//   D:          lane l holds column (l % 32), rows 8*(i/4) + 4*(l/32) + (i%4), i < 16
// The order of the k sum is free, so lane group g = l/32 owns the contiguous
// half [g*d_h/2, (g+1)*d_h/2) of the head dimension. Each lane then reads one
// contiguous half-row of its key (64..256 bytes) with 16-byte loads.
//
// Precision: bf16 keys (and fp8 keys, widened exactly to bf16 in LDS) multiply a
// query split into bf16 hi + lo parts, which keeps about 16 bits of q, with
// fp32 accumulation. fp32 keys use the fp32 MFMA directly.
#pragma once

#include "common.hpp"

namespace lsa {

// ILV: lane group g takes the interleaved 16-byte chunks 2t + g of the head
// dimension (k-step t) instead of the contiguous half [g*d_h/2, (g+1)*d_h/2),
// so that k-steps 0 .. STEPS/2 - 1 use only the first half of every key row.
template <int KT, int DH, int NHB, bool ROT = false, bool ILV = false>
struct Scorer {
  static_assert(DH == 32 || DH == 64 || DH == 128, "d_h");
  static_assert(NHB == 1 || NHB == 2, "heads per block");
  static_assert(!ILV || KT == KEY_BF16, "the interleaved layout is for the split bf16 query");
  static_assert(KT == KEY_F32 || KT == KEY_BF16, "fp8 keys are widened to bf16 before the scorer");
  static constexpr int HALF = DH / 2;                         // k values per lane group
  static constexpr int ESZ = KT == KEY_F32 ? 4 : (KT == KEY_BF16 ? 2 : 1);
  static constexpr int ROW_BYTES = DH * ESZ;
  static constexpr int HALF_BYTES = HALF * ESZ;
  static constexpr int NLD = HALF_BYTES / 16;                 // 16-byte loads per lane
  static constexpr int STEPS = KT == KEY_F32 ? HALF : HALF / 8;  // MFMAs per head block (per part)
  static constexpr bool SPLIT = KT != KEY_F32;

  // query fragments (bf16 hi/lo) or fp32 values
  bf16x8 qa[SPLIT ? NHB : 1][SPLIT ? STEPS : 1][2];
  float qf[SPLIT ? 1 : NHB][SPLIT ? 1 : STEPS];
  float gate[NHB][16];
  // key fragment of the current 32-entry tile
  u32x4 kraw[NLD];

  // Load q[b] and w[b] (fp32) of one (sequence, layer), heads head0 .. head0 + 32*NHB - 1.
  __device__ __forceinline__ void load_query(const float* __restrict__ q, const float* __restrict__ w,
                                             int b, int n_h, int head0 = 0) {
    const int lane = threadIdx.x & 63, g = lane >> 5, n = lane & 31;
#pragma unroll
    for (int mb = 0; mb < NHB; ++mb) {
      const int head = head0 + mb * 32 + n;
      const bool ok = head < n_h;
      const float* qrow = q + ((int64_t)b * n_h + (ok ? head : 0)) * DH + (ILV ? 8 * g : g * HALF);
      if constexpr (SPLIT) {
        constexpr int QS = ILV ? 16 : 8;  // elements between the chunks of consecutive k-steps
#pragma unroll
        for (int t = 0; t < STEPS; ++t) {
          float v[8];
          f32x4 v0 = ok ? *(const f32x4*)(qrow + QS * t) : f32x4{0, 0, 0, 0};
          f32x4 v1 = ok ? *(const f32x4*)(qrow + QS * t + 4) : f32x4{0, 0, 0, 0};
#pragma unroll
          for (int i = 0; i < 4; ++i) { v[i] = v0[i]; v[4 + i] = v1[i]; }
          split8(v, qa[mb][t][0], qa[mb][t][1]);
        }
      } else {
#pragma unroll
        for (int t = 0; t < STEPS; t += 4) {
          f32x4 v = ok ? *(const f32x4*)(qrow + t) : f32x4{0, 0, 0, 0};
#pragma unroll
          for (int i = 0; i < 4; ++i) qf[mb][t + i] = v[i];
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int h = head0 + mb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
        gate[mb][i] = h < n_h ? w[(int64_t)b * n_h + h] : 0.0f;
      }
    }
  }

  // Bound constant of the hi-only score (split query only). A pass that feeds the
  // MFMAs the bf16 hi parts alone computes x_hi; the full pass adds the lo parts
  // to the same accumulators and computes x. For every entry with key K_s,
  //   |x - x_hi| <= sum_j |w_j| (||lo_j|| + 2^-13 ||q_j||) ||K_s|| = C ||K_s||:
  // ReLU is 1-Lipschitz, |lo_j . K_s| <= ||lo_j|| ||K_s|| (Cauchy-Schwarz), and the
  // fp32 rounding of both passes (at most 384 products per dot and 65 gated
  // terms, u = 2^-24) stays below 2^-15 ||q_j|| ||K_s|| per head, which the
  // 2^-13 ||q_j|| term covers four times over. Returns C^2, the same in every
  // lane. Heads at or past n_h have q = 0 and w = 0 and add nothing.
  __device__ __forceinline__ float guard_c2(const float* __restrict__ w, int b, int n_h, int head0 = 0) const {
    static_assert(SPLIT, "the bound needs the split query");
    const int lane = threadIdx.x & 63, n = lane & 31;
    float c = 0.0f;
#pragma unroll
    for (int mb = 0; mb < NHB; ++mb) {
      float sh = 0.0f, sl = 0.0f;
#pragma unroll
      for (int t = 0; t < STEPS; ++t) {
        const u32x4 hv = __builtin_bit_cast(u32x4, qa[mb][t][0]);
        const u32x4 lv = __builtin_bit_cast(u32x4, qa[mb][t][1]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sh = dot2_bf16(hv[i], hv[i], sh);
          sl = dot2_bf16(lv[i], lv[i], sl);
        }
      }
      // lanes l and l ^ 32 hold the two halves of head (head0 + 32 mb + n)
      sh = sum_halves(sh);
      sl = sum_halves(sl);
      const int head = head0 + mb * 32 + n;
      const float wj = head < n_h ? fabsf(w[(int64_t)b * n_h + head]) : 0.0f;
      // hi rounds each element of q to nearest, so ||q_j|| <= ||hi_j|| / (1 - 2^-9) < 1.0117 ||hi_j||
      c += wj * (__builtin_sqrtf(sl) + 0x1.03p-13f * __builtin_sqrtf(sh));
    }
    // sum over the 32 heads of each block: every head is held twice (lanes n and n + 32)
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) c += __shfl_xor(c, o);
    c *= 0.5f;
    // the fp32 sums above round by a relative 2^-17 at most; the margin in the q term covers it
    return __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(c * c)));
  }

  // Load this lane's half of one key row (row pointer already at the half).
  __device__ __forceinline__ void load_keys(const char* __restrict__ p, bool valid) {
#pragma unroll
    for (int i = 0; i < NLD; ++i)
      kraw[i] = valid ? __builtin_nontemporal_load((const u32x4*)p + i) : u32x4{0, 0, 0, 0};
  }

  // Read this lane's half-row of a 32-row tile staged in LDS in the layout of
  // lds_chunk<CPR, ROT>.
  static constexpr int CPR = ROW_BYTES / 16;
  __device__ __forceinline__ void read_keys_lds(const char* tile) {
    const int lane = threadIdx.x & 63, g = lane >> 5, n = lane & 31;
    const char* row = tile + n * ROW_BYTES;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int c = g * (CPR / 2) + i;
      kraw[i] = *(const u32x4*)(row + lds_chunk<CPR, ROT>(c, n) * 16);
    }
  }

  __device__ __forceinline__ void mma(f32x16 (&acc)[NHB]) const {
#pragma unroll
    for (int mb = 0; mb < NHB; ++mb) acc[mb] = f32x16{};
    if constexpr (KT == KEY_BF16) {
#pragma unroll
      for (int t = 0; t < STEPS; ++t) {
        const bf16x8 kb = as_bf16x8(kraw[t]);
#pragma unroll
        for (int mb = 0; mb < NHB; ++mb) {
          acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[mb][t][0], kb, acc[mb], 0, 0, 0);
          acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[mb][t][1], kb, acc[mb], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < STEPS; ++t) {
        const float kv = __uint_as_float(kraw[t >> 2][t & 3]);
#pragma unroll
        for (int mb = 0; mb < NHB; ++mb)
          acc[mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(qf[mb][t], kv, acc[mb], 0, 0, 0);
      }
    }
  }

  // Gate, ReLU and head sum. Lanes l and l^32 hold complementary heads of the
  // same entry. After one swap both lanes have the full sum. Addition is
  // commutative, so both lanes hold the identical value. The ReLU is
  // max(int(x), 0) on the float's bits: exact for IEEE floats (every negative
  // value, -0 included, becomes +0) and free of NaN canonicalisation.
  // This lane's share of the head sum (its 16*NHB heads), before the lane swap.
  // Two interleaved sums halve the dependent chain of FMAs.
  __device__ __forceinline__ float partial(const f32x16 (&acc)[NHB]) const {
    float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
    for (int mb = 0; mb < NHB; ++mb)
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        p0 = fmaf(gate[mb][i], __int_as_float(max(__float_as_int(acc[mb][i]), 0)), p0);
        p1 = fmaf(gate[mb][i + 1], __int_as_float(max(__float_as_int(acc[mb][i + 1]), 0)), p1);
      }
    return p0 + p1;
  }

  __device__ __forceinline__ float logit(const f32x16 (&acc)[NHB]) const {
    float part = 0.0f;
#pragma unroll
    for (int mb = 0; mb < NHB; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        part = fmaf(gate[mb][i], __int_as_float(max(__float_as_int(acc[mb][i]), 0)), part);
    return part + __shfl_xor(part, 32);
  }
};

}  // namespace lsa
