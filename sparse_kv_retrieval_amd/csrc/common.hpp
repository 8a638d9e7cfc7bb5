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

// ------------------------------------------------------------- e4m3fn -> bf16
// Exact widening of 4 OCP e4m3fn bytes (one dword) to 4 bfloat16 values (two
// dwords). For exponent field e >= 1 the value is 2^(e-7) (1 + m/8). Placing
// the 7 exponent/mantissa bits at float32 bit 20 gives 2^(e-127) (1 + m/8),
// and multiplying by 2^120 rescales it exactly. Subnormal bytes (e = 0) become
// float32 subnormals m/8 2^-126, and the same multiply gives m 2^-9. Every
// result has at most 4 significant bits, so truncating to the high half is
// exact. Finite inputs only: the NaN byte is not a valid key.
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t two) {
  // `two` holds two bytes in bits 0..7 and 8..15.
  float f0 = __uint_as_float((two & 0x7Fu) << 20) * 0x1p120f;
  float f1 = __uint_as_float(((two >> 8) & 0x7Fu) << 20) * 0x1p120f;
  uint32_t b0 = (__float_as_uint(f0) >> 16) | ((two & 0x80u) << 8);
  uint32_t b1 = (__float_as_uint(f1) >> 16) | (((two >> 8) & 0x80u) << 8);
  return b0 | (b1 << 16);
}

__device__ __forceinline__ u32x2 e4m3x4_to_bf16x4(uint32_t four) {
  u32x2 r;
  r[0] = e4m3x2_to_bf16x2(four & 0xFFFFu);
  r[1] = e4m3x2_to_bf16x2(four >> 16);
  return r;
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
