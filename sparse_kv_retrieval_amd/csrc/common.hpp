// Shared device helpers for the gfx950 kernels of the LSA selection path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lsa.h"

namespace lsa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum KeyKind { KEY_F32 = 0, KEY_BF16 = 1, KEY_FP8 = 2 };

// ---------------------------------------------------------------- bf16 bits
// Round-to-nearest-even float -> bfloat16 bits. Inputs here are finite.
__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Split 8 fp32 values into bfloat16 hi + lo with x ~= hi + lo (about 16
// significant bits). Both halves are packed as MFMA operands.
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
  u32x4 h, l;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t h0 = bf16_rne_bits(x[2 * i]), h1 = bf16_rne_bits(x[2 * i + 1]);
    uint32_t l0 = bf16_rne_bits(x[2 * i] - bf16_bits_to_f32(h0));
    uint32_t l1 = bf16_rne_bits(x[2 * i + 1] - bf16_bits_to_f32(h1));
    h[i] = h0 | (h1 << 16);
    l[i] = l0 | (l1 << 16);
  }
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, l);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// c + a.lo * b.lo + a.hi * b.hi for two packed bfloat16 pairs (v_dot2_f32_bf16).
// bf16 products are exact in fp32; the sum rounds once or twice.
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// ------------------------------------------------------------- e4m3fn -> bf16
// Widening of 4 OCP e4m3fn bytes (one dword) to 4 bfloat16 values (two
// dwords, byte i -> element i) with the gfx950 conversion instruction
// (v_cvt_scalef32_pk_bf16_fp8, scale 1). Every finite e4m3fn value has at most
// 4 significant bits and an exponent in [-9, 8], so bf16 holds it exactly; a
// one-launch check over all 256 codes matched the format's definition.
// Finite inputs only: the NaN byte is not a valid key.
__device__ __forceinline__ u32x2 e4m3x4_to_bf16x4(uint32_t four) {
  u32x2 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(four, 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(four, 1.0f, true));
  return r;
}

// ------------------------------------------------------------- buffer loads
// Raw buffer resource over [base, base + bytes). A load at an offset >= bytes
// returns zeros without a memory access. The streaming kernels use this to
// issue the same loads on every path: a slot with nothing to fetch (past the
// end of a wave's work, or the tail of a ragged tile) gets an out-of-range
// offset instead of a branch. The compiler's wait counts then stay exact, and
// no wait drains the loads still in flight. Callers keep bytes < 2^31.
constexpr uint32_t BUF_OOB = 0x80000000u;
constexpr int BUF_NT = 2;  // cache policy: non-temporal

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, BUF_NT));
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}

// ------------------------------------------------------------- LDS tile layout
// Position of 16-byte chunk c of row r in a 32-row tile staged in LDS, with
// CPR chunks per row. Rows are XOR-swizzled (chunk c of row r at c ^ (r % CPR))
// so that 8 lanes reading the same chunk of 8 consecutive rows hit 8 distinct
// 16-byte bank groups. With ROT the chunk index is first rotated right by one
// bit, c -> (c >> 1) | ((c & 1) * CPR / 2). This is for fp8 tiles, where each
// lane writes the two LDS chunks 2j and 2j + 1 that one 16-byte load widens
// to, and 8 lanes write chunks 2j, j = 0..7, of one row. Rotated, those land
// on 8 distinct bank groups too.
template <int CPR, bool ROT>
__device__ __forceinline__ int lds_chunk(int c, int r) {
  if constexpr (ROT) c = (c >> 1) | ((c & 1) * (CPR / 2));
  return c ^ (r % CPR);
}

// Sum of a lane's value and the value of lane l ^ 32 (the other half of the
// wave), in both halves. v_permlane32_swap exchanges the upper half of one
// register with the lower half of the other, so with both operands equal to x
// the two results hold x[l] and x[l ^ 32] at every lane; the add is the same
// low-half + high-half sum in both halves.
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Values the whole wave agrees on, pinned to scalar registers. Loads from memory
// are vector loads, and without this the compiler keeps their results (and
// everything derived from them) in VGPRs.
__device__ __forceinline__ int32_t uni(int32_t x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uni(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// ----------------------------------------------------------------- search
// Largest b in [0, n) with off[b] <= x, given off[0] <= x < off[n] and off
// non-decreasing. It also skips over empty sequences (off[b] == off[b+1]).
template <typename T>
__device__ __forceinline__ int upper_seq(const T* off, int n, T x) {
  int lo = 0, hi = n;  // invariant: off[lo] <= x < off[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (off[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

// Order-preserving map of a finite float to uint32 (ascending float ->
// ascending key). -0.0 is folded into +0.0 first, so the two compare equal.
__device__ __forceinline__ uint32_t order_key(float y) {
  uint32_t u = __float_as_uint(y + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace lsa
