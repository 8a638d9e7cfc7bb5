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
//   mode 2: as mode 1, with non-temporal loads;
//   mode 3: each wave reads its own contiguous range straight into an LDS
//           ring (buffer_load ... lds, non-temporal), four 4 KiB slots per
//           wave and 8 waves per block, and reads every slot back from LDS
//           before refilling it: the memory path of the key scan, without
//           its arithmetic. `blocks` is then the number of 512-thread blocks.
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

template <int RU>
__global__ __launch_bounds__(512) void probe_lds_ring(const char* __restrict__ p, int64_t bytes,
                                                      uint32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(1024))) char ring[8][RU][4096];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nunits = (bytes + 4095) / 4096;
  const int64_t nw = (int64_t)gridDim.x * 8, gw = (int64_t)blockIdx.x * 8 + w;
  const int64_t u0 = gw * nunits / nw, u1 = (gw + 1) * nunits / nw;
  // bytes < 2^31 (checked by the host): an offset at or past it reads zeros without a memory access
  const auto r = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p), (short)0, (int)bytes, 0x00020000);
  constexpr uint32_t OOB = 0x80000000u;
  auto issue = [&](int64_t u, int slot) {
    const uint32_t off = u < u1 ? (uint32_t)(u * 4096) : OOB;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)&ring[w][slot][k * 1024],
                                               16, off + k * 1024 + lane * 16, 0, 0, 2);
  };
#pragma unroll
  for (int s = 0; s < RU; ++s) issue(u0 + s, s);
  uint32_t acc = 0;
  int slot = 0;
  for (int64_t u = u0; u < u1; ++u) {
    // unit u has landed once at most the RU - 1 later units' loads are outstanding
    __builtin_amdgcn_s_waitcnt((((RU - 1) * 4) & 15) | ((((RU - 1) * 4) >> 4) << 14) | (7 << 4) | (15 << 8));
    asm volatile("" ::: "memory");
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      u32x4p v;
      const uint32_t a = (uint32_t)(size_t)(const __attribute__((address_space(3))) void*)&ring[w][slot][k * 1024 + lane * 16];
      asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
      acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    issue(u + RU, slot);
    slot = slot + 1 == RU ? 0 : slot + 1;
  }
  // no load may still be writing LDS when the wave ends
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
  if (lane == 0) atomicXor(sink + blockIdx.x, acc);
}

// sink: blocks words of device memory. Returns 0, -1 for bad arguments, -3 for a launch error.
extern "C" int probe_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int32_t blocks, int32_t mode,
                                 int32_t loads_in_flight, hipStream_t st) {
  if (!buf || !sink || bytes < 16 || (bytes & 15) || ((uintptr_t)buf & 15) || blocks < 1) return -1;
  if (mode < 0 || mode > 3 || (loads_in_flight != 8 && loads_in_flight != 16)) return -1;
  if (mode == 3) {
    if (bytes >= (int64_t)1 << 31) return -1;
    hipLaunchKernelGGL(probe_lds_ring<4>, dim3(blocks), dim3(512), 0, st, (const char*)buf, bytes, sink);
    return hipGetLastError() == hipSuccess ? 0 : -3;
  }
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
