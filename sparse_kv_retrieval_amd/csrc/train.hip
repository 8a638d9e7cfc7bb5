// One training step of a memory-indexer layer: loss and gradients of W^DQ,
// W^IUQ and W^w against frozen keys.
//
// marsggbo write-up, "4. 训练" (training), and the hyper.ai digest, "方法"
// (Method): the compressed index keys are precomputed and fixed, and only the
// query side's projections are trained, with binary cross-entropy made focal
// (the gist.science summary states the same loss). The score is the
// selection path's: I_s = sigmoid(x_s), x_s = sum_j w_j ReLU(q_j . K_s),
// q = (h W^DQ) W^IUQ, w = h W^w ([BLOG] §3.1). Focal form with p = I_s:
// -alpha (1-p)^gamma log p for a golden entry, -(1-alpha) p^gamma log(1-p)
// otherwise; the loss is the mean over the batch's entries.
//
// Kernels, after the projection kernels give c, q and w:
//   train_scan_kernel  one pass over the keys (4 waves per block, 16 heads per
//                      wave, tiles of 32 entries staged in LDS twice: row-major
//                      for the score MFMAs and transposed for the gradient
//                      MFMAs). Per tile: the head dots S = K q^T on bf16 MFMA
//                      (q split hi + lo), x_s, the loss, g_s = dloss/dx_s, and
//                      the contraction dq_j += sum_s g_s w_j [S_sj > 0] K_s on
//                      MFMA (coefficients split hi + lo), dw_j += sum_s g_s
//                      ReLU(S_sj). Per-block partial sums go to the workspace.
//   train_reduce_kernel  sums a sequence's block partials: dq, dw, the loss.
//   train_dc_kernel    dc = dq W^IUQ (bf16 weights), per row block, and
//   sum kernel         the row blocks' partials added.
//   train_outer_kernel rank-B products for the three gradients:
//                      g_iuq = dq^T c, g_dq = dc^T h, g_w = dw^T h.
#include "kernels.hpp"

namespace lsa {

namespace {

constexpr int TT = 256;            // scan block: 4 waves
constexpr int TNH = 64;            // heads (16 per wave)
constexpr int TDH = 128;           // head dim = key dim
constexpr int TE = 32;             // entries per tile
constexpr int TPB = 32;            // tiles per scan block
constexpr int BE = TE * TPB;       // entries per scan block
constexpr int PW = TNH * TDH + TNH + 1;  // floats per block partial: dq, dw, loss
constexpr float TLOG2E = 1.4426950408889634f;

struct TrainScanSmem {
  uint4 kt[TE * 16];               // tile row-major: chunk c of entry e at e*16 + (c ^ (e & 15))
  uint32_t ktt[TDH * TE / 2];      // tile transposed: entry e of dim d at byte d*64 + ((e/8) ^ ((d/2)&3))*16 + (e%8)*2
  float xpart[4][TE];
  uint32_t coef[4][2][16][TE / 2]; // per wave: hi and lo bf16 of d loss / d S, [head][entry]
  double lsum[4];
};

__device__ __forceinline__ float t_log_sigmoid(float x) {  // log(1 / (1 + exp(-x))), stable for both signs
  return fminf(x, 0.f) - log1pf(__expf(-fabsf(x)));
}

// Focal loss term and its derivative in the logit x (fp32), label y.
__device__ __forceinline__ void focal(float x, bool y, float gamma, float alpha, float& loss, float& grad) {
  const float lp = t_log_sigmoid(x), lq = t_log_sigmoid(-x);  // log p, log(1 - p)
  const float p = __expf(lp), q = __expf(lq);
  if (y) {
    const float qg = gamma == 0.f ? 1.f : powf(q, gamma);
    loss = -alpha * qg * lp;
    grad = alpha * qg * (gamma * p * lp - q);
  } else {
    const float pg = gamma == 0.f ? 1.f : powf(p, gamma);
    loss = -(1.f - alpha) * pg * lq;
    grad = (1.f - alpha) * pg * (p - gamma * q * lq);
  }
}

__device__ __forceinline__ uint32_t pack_bf16x2(uint32_t lo, uint32_t hi) { return lo | (hi << 16); }

// First scan block of sequence b (blocks are laid out sequence by sequence).
__device__ __forceinline__ int64_t first_block(const int64_t* __restrict__ off, int b) {
  int64_t s = 0;
  for (int i = 0; i < b; ++i) s += (off[i + 1] - off[i] + BE - 1) / BE;
  return s;
}

__global__ __launch_bounds__(TT) void train_scan_kernel(const TrainArgs a) {
  __shared__ TrainScanSmem sm;
  const int t = threadIdx.x, lane = t & 63;
  const int wq = __builtin_amdgcn_readfirstlane(t >> 6);
  const int hl = lane & 15, kg = lane >> 4;
  // this block's sequence and entry range
  int b = 0;
  int64_t blk0 = 0;
  for (;; ++b) {
    const int64_t nb = (a.key_off[b + 1] - a.key_off[b] + BE - 1) / BE;
    if ((int64_t)blockIdx.x < blk0 + nb) break;
    blk0 += nb;
  }
  const int64_t n_b = a.key_off[b + 1] - a.key_off[b];
  const int64_t e_begin = ((int64_t)blockIdx.x - blk0) * BE;
  const int ntiles = (int)min((int64_t)TPB, (n_b - e_begin + TE - 1) / TE);
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
  float dwl = 0.f;
  double ll = 0.0;

  // tile loads: thread t holds chunks 2c, 2c+1 (16 bf16) of entry t / 8
  const int le = t >> 3, lc = (t & 7) * 2;
  auto load_tile = [&](int tile, u32x4& v0, u32x4& v1) {
    const uint32_t off = (uint32_t)((e_begin + (int64_t)tile * TE + le) * (TDH * 2) + lc * 16);
    v0 = buf_load16(rs, off);
    v1 = buf_load16(rs, off + 16);
  };
  u32x4 n0, n1;
  load_tile(0, n0, n1);
  for (int tile = 0; tile < ntiles; ++tile) {
    const u32x4 c0 = n0, c1 = n1;
    if (tile + 1 < ntiles) load_tile(tile + 1, n0, n1);
    const int64_t s0 = e_begin + (int64_t)tile * TE;  // first entry of the tile (a multiple of 32)
    // ---- stage the tile: row-major (swizzled) and transposed
    sm.kt[le * 16 + (lc ^ (le & 15))] = __builtin_bit_cast(uint4, c0);
    sm.kt[le * 16 + ((lc + 1) ^ (le & 15))] = __builtin_bit_cast(uint4, c1);
    {
      uint16_t* tt = (uint16_t*)sm.ktt;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t w32 = j < 4 ? c0[j] : c1[j - 4];
#pragma unroll
        for (int hlf = 0; hlf < 2; ++hlf) {
          const int d = lc * 8 + 2 * j + hlf;
          tt[(d * 64 + (((le >> 3) ^ ((d >> 1) & 3)) * 16) + (le & 7) * 2) / 2] = (uint16_t)(w32 >> (16 * hlf));
        }
      }
    }
    __syncthreads();
    // ---- head dots of 32 entries x this wave's 16 heads
    f32x4 S[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const int e = 16 * mb + hl;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 A = __builtin_bit_cast(bf16x8, sm.kt[e * 16 + ((4 * ks + kg) ^ (e & 15))]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, qh[ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, ql[ks], acc, 0, 0, 0);
      }
      S[mb] = acc;  // S[mb][i]: entry 16mb + 4kg + i, head 16wq + hl
    }
    // partial x over this wave's heads, summed over the 16 lanes of each group
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = wh * fmaxf(S[mb][i], 0.f);
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o);
        if (hl == 0) sm.xpart[wq][16 * mb + 4 * kg + i] = v;
      }
    __syncthreads();
    // ---- loss, d loss / d x, the gate gradient and the coefficients d loss / d S
    const uint32_t lw = (uint32_t)(lab[s0 >> 6] >> (s0 & 63));  // the tile's 32 labels
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      uint32_t hi2[2] = {0, 0}, lo2[2] = {0, 0};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 16 * mb + 4 * kg + i;
        const float x = sm.xpart[0][e] + sm.xpart[1][e] + sm.xpart[2][e] + sm.xpart[3][e];
        const bool valid = s0 + e < n_b;
        float fl, fg;
        focal(x, (lw >> e) & 1, a.gamma, a.alpha, fl, fg);
        const float g = valid ? fg * a.inv_total : 0.f;
        if (valid && wq == 0 && hl == 0) ll += (double)fl;
        dwl += g * fmaxf(S[mb][i], 0.f);
        const float cf = S[mb][i] > 0.f ? g * wh : 0.f;
        const uint32_t h16 = bf16_rne_bits(cf);
        const uint32_t l16 = bf16_rne_bits(cf - bf16_bits_to_f32(h16));
        if (i & 1) {
          hi2[i >> 1] |= h16 << 16;
          lo2[i >> 1] |= l16 << 16;
        } else {
          hi2[i >> 1] = h16;
          lo2[i >> 1] = l16;
        }
      }
      const int wi = (16 * mb + 4 * kg) / 2;
      *(uint2*)&sm.coef[wq][0][hl][wi] = make_uint2(hi2[0], hi2[1]);
      *(uint2*)&sm.coef[wq][1][hl][wi] = make_uint2(lo2[0], lo2[1]);
    }
    // ---- dq for this wave's heads: coef^T (16 heads x 32 entries) x K (32 entries x 128)
    __builtin_amdgcn_wave_barrier();  // coef is written and read by this wave only: LDS keeps the wave's order
    {
      const bf16x8 Ah = __builtin_bit_cast(bf16x8, *(const uint4*)&sm.coef[wq][0][hl][4 * kg]);
      const bf16x8 Al = __builtin_bit_cast(bf16x8, *(const uint4*)&sm.coef[wq][1][hl][4 * kg]);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const int d = 16 * nb + hl;
        const bf16x8 Bk = __builtin_bit_cast(bf16x8, *(const uint4*)((const char*)sm.ktt + d * 64 + ((kg ^ ((d >> 1) & 3)) * 16)));
        accb[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ah, Bk, accb[nb], 0, 0, 0);
        accb[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Al, Bk, accb[nb], 0, 0, 0);
      }
    }
    __syncthreads();  // the next tile overwrites kt and ktt
  }

  // ---- this block's partial sums
  float* part = a.part + (int64_t)blockIdx.x * PW;
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) part[(16 * wq + 4 * kg + i) * TDH + 16 * nb + hl] = accb[nb][i];
  dwl += __shfl_xor(dwl, 16);
  dwl += __shfl_xor(dwl, 32);
  if (kg == 0) part[TNH * TDH + 16 * wq + hl] = dwl;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ll += __shfl_xor(ll, o);
  if (lane == 0) sm.lsum[wq] = ll;
  __syncthreads();
  if (t == 0) part[TNH * TDH + TNH] = (float)(sm.lsum[0] + sm.lsum[1] + sm.lsum[2] + sm.lsum[3]);
}

// dq[b], dw[b] = sums of sequence b's block partials; the loss from every block.
__global__ __launch_bounds__(256) void train_reduce_kernel(const TrainArgs a) {
  const int b = blockIdx.y;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= PW) return;
  if (j == PW - 1) {  // the loss: every block of every sequence, once
    if (b == 0) {
      double s = 0.0;
      for (int64_t k = 0; k < a.nblk; ++k) s += (double)a.part[k * PW + PW - 1];
      a.loss[0] = (float)(s * (double)a.inv_total);
    }
    return;
  }
  const int64_t k0 = first_block(a.key_off, b);
  const int64_t k1 = k0 + (a.key_off[b + 1] - a.key_off[b] + BE - 1) / BE;
  float s = 0.f;
  for (int64_t k = k0; k < k1; ++k) s += a.part[k * PW + j];
  if (j < TNH * TDH)
    a.dq[(int64_t)b * TNH * TDH + j] = s;
  else
    a.dw[(int64_t)b * TNH + (j - TNH * TDH)] = s;
}

// Partial dc over 64 rows o of W^IUQ: dcp[blk][b][k] = sum_o dq[b][o] W[o][k].
// Thread t owns columns 8t..8t+7 of a 2048-column chunk (blockIdx.y).
constexpr int DCR = 64;
__global__ __launch_bounds__(256) void train_dc_kernel(const TrainArgs a) {
  __shared__ float dqs[DCR][32];
  const int o0 = blockIdx.x * DCR;
  const int k = blockIdx.y * 2048 + threadIdx.x * 8;
  for (int i = threadIdx.x; i < DCR * a.B; i += 256) dqs[i % DCR][i / DCR] = a.dq[(int64_t)(i / DCR) * TNH * TDH + o0 + i % DCR];
  __syncthreads();
  if (k >= a.r) return;
  const uint16_t* W = (const uint16_t*)a.w_iuq;
  for (int b0 = 0; b0 < a.B; b0 += 8) {
    float acc[8][8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[u][c] = 0.f;
    for (int o = 0; o < DCR; ++o) {
      const uint4 raw = *(const uint4*)(W + (int64_t)(o0 + o) * a.r + k);
      float wv[8];
      const uint32_t rw[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        wv[2 * c] = bf16_bits_to_f32(rw[c] & 0xFFFFu);
        wv[2 * c + 1] = bf16_bits_to_f32(rw[c] >> 16);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float dv = b0 + u < a.B ? dqs[o][b0 + u] : 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[u][c] = fmaf(dv, wv[c], acc[u][c]);
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (b0 + u < a.B)
#pragma unroll
        for (int c = 0; c < 8; ++c) a.dcp[((int64_t)blockIdx.x * a.B + b0 + u) * a.r + k + c] = acc[u][c];
  }
}

// out[i] = sum over p < nparts of in[p * n + i]
__global__ __launch_bounds__(256) void train_sum_kernel(const float* __restrict__ in, int nparts, int64_t n,
                                                      float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int p = 0; p < nparts; ++p) s += in[(int64_t)p * n + i];
  out[i] = s;
}

// out[i][j] = sum_b u[b][i] v[b][j] (u fp32 with row stride I, v fp32 or bf16 with row stride J).
// Block: 32 rows i x 256 columns j, one column per thread.
template <bool VBF16>
__global__ __launch_bounds__(256) void train_outer_kernel(const float* __restrict__ u, const void* __restrict__ v,
                                                        int B, int64_t I, int64_t J, float* __restrict__ out) {
  __shared__ float us[32][32];  // [b][i]
  const int64_t i0 = (int64_t)blockIdx.y * 32;
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (int x = threadIdx.x; x < 32 * 32; x += 256) {  // rows b >= B are zero: garbage times zero may be NaN
    const int bb = x / 32, ii = x % 32;
    us[bb][ii] = bb < B && i0 + ii < I ? u[(int64_t)bb * I + i0 + ii] : 0.f;
  }
  __syncthreads();
  if (j >= J) return;
  float vb[32];
#pragma unroll
  for (int bb = 0; bb < 32; ++bb) {
    float x = 0.f;
    if (bb < B) {
      if constexpr (VBF16)
        x = bf16_bits_to_f32(((const uint16_t*)v)[(int64_t)bb * J + j]);
      else
        x = ((const float*)v)[(int64_t)bb * J + j];
    }
    vb[bb] = x;
  }
  for (int ii = 0; ii < 32 && i0 + ii < I; ++ii) {
    float s = 0.f;
#pragma unroll
    for (int bb = 0; bb < 32; ++bb) s = fmaf(us[bb][ii], vb[bb], s);
    out[(i0 + ii) * J + j] = s;
  }
}

}  // namespace

int64_t train_scan_blocks(const int64_t* key_off_host, int B) {
  int64_t s = 0;
  for (int b = 0; b < B; ++b) s += (key_off_host[b + 1] - key_off_host[b] + BE - 1) / BE;
  return s;
}

size_t train_workspace_bytes(int B, int r, int64_t nblk) {
  const int64_t f = (int64_t)B * r * 2 + (int64_t)B * TNH * TDH * 2 + (int64_t)B * TNH * 2 + nblk * PW +
                    (int64_t)(TNH * TDH / DCR) * B * r;
  return (size_t)f * 4 + 256;
}

hipError_t launch_train(const TrainArgs& a, hipStream_t st) {
  hipError_t e;
  if (a.nblk > 0) {
    hipLaunchKernelGGL(train_scan_kernel, dim3((unsigned)a.nblk), dim3(TT), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(train_reduce_kernel, dim3((PW + 255) / 256, a.B), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int nrb = TNH * TDH / DCR;
  hipLaunchKernelGGL(train_dc_kernel, dim3(nrb, (a.r + 2047) / 2048), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t ndc = (int64_t)a.B * a.r;
  hipLaunchKernelGGL(train_sum_kernel, dim3((unsigned)((ndc + 255) / 256)), dim3(256), 0, st, a.dcp, nrb, ndc, a.dc);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // g_iuq = dq^T c, g_dq = dc^T h, g_w = dw^T h
  hipLaunchKernelGGL(train_outer_kernel<false>, dim3((a.r + 255) / 256, (TNH * TDH + 31) / 32), dim3(256), 0, st,
                     a.dq, (const void*)a.c, a.B, (int64_t)TNH * TDH, (int64_t)a.r, a.g_iuq);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(train_outer_kernel<true>, dim3((a.d + 255) / 256, (a.r + 31) / 32), dim3(256), 0, st, a.dc,
                     a.h, a.B, (int64_t)a.r, (int64_t)a.d, a.g_dq);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(train_outer_kernel<true>, dim3((a.d + 255) / 256, (TNH + 31) / 32), dim3(256), 0, st, a.dw,
                     a.h, a.B, (int64_t)TNH, (int64_t)a.d, a.g_w);
  return hipGetLastError();
}

}  // namespace lsa
