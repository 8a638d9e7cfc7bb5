// Streaming-read reference for the rooflines (measurement only; not part of
// the selection path and not declared in lsa.h).
//
// probe_stream_read reads `bytes` of device memory once with 16-byte loads and
// folds what it read into one word per block, so the loads cannot be dropped.
// It is the plainest way to read HBM: its rate is the ceiling that a kernel
// streaming the same number of bytes (the key scan) is compared with. The
// access pattern is a parameter, and the caller takes the fastest:
//   mode 0: grid-stride loop, U loads in flight per thread;
//   mode 1: each block reads its own contiguous range (as the score pass
//           does), U loads in flight per thread;
//   mode 2: as mode 1, with non-temporal loads.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4p __attribute__((ext_vector_type(4)));

template <int U, bool NT>
__device__ __forceinline__ u32x4p ld(const u32x4p* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

template <int U>
__global__ __launch_bounds__(256) void probe_grid_stride(const u32x4p* __restrict__ p, int64_t n16,
                                                         uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4p v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4p v = p[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) atomicXor(sink + blockIdx.x, acc);
}

template <int U, bool NT>
__global__ __launch_bounds__(256) void probe_block_range(const u32x4p* __restrict__ p, int64_t n16,
                                                         uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t lo = (int64_t)blockIdx.x * n16 / gridDim.x, hi = ((int64_t)blockIdx.x + 1) * n16 / gridDim.x;
  constexpr int T = 256;
  int64_t i = lo + threadIdx.x;
  for (; i + (U - 1) * T < hi; i += U * T) {
    u32x4p v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = ld<U, NT>(p + i + u * T);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < hi; i += T) {
    const u32x4p v = ld<U, NT>(p + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) atomicXor(sink + blockIdx.x, acc);
}

// sink: blocks words of device memory. Returns 0, -1 for bad arguments, -3 for a launch error.
extern "C" int probe_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int32_t blocks, int32_t mode,
                                 int32_t loads_in_flight, hipStream_t st) {
  if (!buf || !sink || bytes < 16 || (bytes & 15) || ((uintptr_t)buf & 15) || blocks < 1) return -1;
  if (mode < 0 || mode > 2 || (loads_in_flight != 8 && loads_in_flight != 16)) return -1;
  const u32x4p* p = (const u32x4p*)buf;
  const int64_t n = bytes / 16;
  const bool u16 = loads_in_flight == 16;
  if (mode == 0) {
    if (u16) hipLaunchKernelGGL(probe_grid_stride<16>, dim3(blocks), dim3(256), 0, st, p, n, sink);
    else hipLaunchKernelGGL(probe_grid_stride<8>, dim3(blocks), dim3(256), 0, st, p, n, sink);
  } else if (mode == 1) {
    if (u16) hipLaunchKernelGGL((probe_block_range<16, false>), dim3(blocks), dim3(256), 0, st, p, n, sink);
    else hipLaunchKernelGGL((probe_block_range<8, false>), dim3(blocks), dim3(256), 0, st, p, n, sink);
  } else {
    if (u16) hipLaunchKernelGGL((probe_block_range<16, true>), dim3(blocks), dim3(256), 0, st, p, n, sink);
    else hipLaunchKernelGGL((probe_block_range<8, true>), dim3(blocks), dim3(256), 0, st, p, n, sink);
  }
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
