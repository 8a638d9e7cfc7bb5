// Score + threshold over every compressed entry, one wave per 32-entry tile.
//
// Same computation as score_select_kernel (the lookahead index score and its
// loading rule, [BLOG] §3.1 of the FlashMemory-DeepSeek-V4 write-up:
// I = sigma(sum_j w_j ReLU(q_j . K_s)), entries with I >= 0.5 are loaded), with
// a different split of the work for bf16 and fp8 keys:
//
//  - Each wave scores all heads of its own tiles, so no tile is shared between
//    waves: there is no barrier and no exchange of partial sums.
//  - Keys go from HBM straight into LDS (buffer_load ... lds). No registers
//    hold keys in flight, and no instruction copies them into LDS.
//  - The LDS holds a ring of RU half tiles (16 key rows each). A tile is two
//    consecutive half tiles. As soon as the wave has read tile j out of LDS,
//    it issues the loads of tile j + RU/2 into the slots tile j leaves, so
//    while it scores tile j the loads of the next RU/2 tiles are in flight.
//
// A block is the WPB waves of one CU. It owns a contiguous run of mask words
// (64 entries, two tiles each), cut into chunks of a few words, and its waves
// take chunks from a counter in LDS whenever they finish one. Two waves on one
// SIMD progress at quite different speeds (the older one wins the issue
// arbitration); with a static split per wave the slower one would set the
// block's time. A claim is an LDS round trip that never waits on the key
// loads. A wave reloads its query only when its words cross into another
// (layer, sequence).
//
// LDS layout of a half tile: its rows are contiguous in HBM, and so in 256-byte
// lines. The 16-byte chunk at position p of line L holds the chunk p ^ (L % 16)
// of that line in HBM. A load instruction writes 1 KiB of LDS in lane order,
// so each lane loads the HBM chunk that belongs at its LDS position. The
// operand reads (16 lanes, 16 rows, one chunk column) then touch 16 distinct
// chunk positions, free of bank conflicts, for every row size from 64 to 256
// bytes.
#include "kernels.hpp"
#include "scorer.hpp"
#include "cursor.hpp"

namespace lsa {

#define LSA_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// Load of 16 (or 4) bytes per lane from a buffer straight into LDS: lane i
// writes LDS bytes [lds + SZ*i, lds + SZ*(i+1)).
__device__ __forceinline__ void dma_lds16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, LSA_LDS(lds), 16, off, 0, 0, BUF_NT);
}
__device__ __forceinline__ void dma_lds4(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, LSA_LDS(lds), 4, off, 0, 0, 0);
}

// HBM offset <-> LDS offset of a 16-byte chunk within a half tile (an involution).
__host__ __device__ constexpr uint32_t stream_swz(uint32_t off) {
  return (off & ~255u) | ((((off >> 4) ^ (off >> 8)) & 15u) << 4);
}

// s_waitcnt vmcnt(N), other counters untouched (gfx9 encoding).
template <int N>
__device__ __forceinline__ void stream_vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

// 32-bit LDS address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) void*)p;
}

// Operand reads of LDS that the key loads (buffer_load ... lds) wrote. The
// compiler does not track which of those loads a read depends on, so for a
// plain LDS read it would first wait for every load in flight (vmcnt(0)) and
// drain the ring. The kernel waits for exactly the loads of the tile it reads
// (stream_vm_wait), and these reads are issued from one asm block that also
// waits for their own results (lgkmcnt(0)) before it ends. With SC, a 4-byte
// read at sa is added (the fp8 scale of the lane's entry).
#define LSA_RD(i, j) "ds_read_b128 %" #i ", %" #j "\n\t"
template <int N, bool SC>
__device__ __forceinline__ void lds_read_tile(u32x4 (&r)[N], const uint32_t (&ad)[N], uint32_t sa, float& sc) {
  static_assert(N == 2 || N == 4 || N == 8, "chunks per lane");
  if constexpr (N == 8 && !SC) {
    asm volatile(LSA_RD(0, 8) LSA_RD(1, 9) LSA_RD(2, 10) LSA_RD(3, 11) LSA_RD(4, 12) LSA_RD(5, 13) LSA_RD(6, 14)
                 LSA_RD(7, 15) "s_waitcnt lgkmcnt(0)"
                 : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
                 : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]), "v"(ad[7])
                 : "memory");
  } else if constexpr (N == 4 && !SC) {
    asm volatile(LSA_RD(0, 4) LSA_RD(1, 5) LSA_RD(2, 6) LSA_RD(3, 7) "s_waitcnt lgkmcnt(0)"
                 : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
                 : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
                 : "memory");
  } else if constexpr (N == 2 && !SC) {
    asm volatile(LSA_RD(0, 2) LSA_RD(1, 3) "s_waitcnt lgkmcnt(0)"
                 : "=&v"(r[0]), "=&v"(r[1])
                 : "v"(ad[0]), "v"(ad[1])
                 : "memory");
  } else if constexpr (N == 4 && SC) {
    asm volatile(LSA_RD(0, 5) LSA_RD(1, 6) LSA_RD(2, 7) LSA_RD(3, 8) "ds_read_b32 %4, %9\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(sc)
                 : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(sa)
                 : "memory");
  } else if constexpr (N == 2 && SC) {
    asm volatile(LSA_RD(0, 3) LSA_RD(1, 4) "ds_read_b32 %2, %5\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(r[0]), "=&v"(r[1]), "=&v"(sc)
                 : "v"(ad[0]), "v"(ad[1]), "v"(sa)
                 : "memory");
  } else {
    static_assert(N == 0, "no such read shape");
  }
}
#undef LSA_RD

// MFMA B operand of k-step s from a lane's half row read out of LDS: bf16 keys
// as they are; fp8 keys (half (s & 1) of chunk s / 2) widened exactly to bf16.
template <int KT, int NCH>
__device__ __forceinline__ bf16x8 key_step_t(const u32x4 (&kr)[NCH], int s) {
  if constexpr (KT == KEY_BF16) {
    return as_bf16x8(kr[s]);
  } else {
    const u32x4& c = kr[s >> 1];
    const u32x2 lo = e4m3x4_to_bf16x4(c[2 * (s & 1)]), hi = e4m3x4_to_bf16x4(c[2 * (s & 1) + 1]);
    return as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
  }
}

// Atomic increment of an LDS counter, returning the old value. From an asm
// block for the same reason as the reads above (a plain LDS atomic would
// first wait for every load in flight); the block waits for its own result.
__device__ __forceinline__ uint32_t lds_fetch_inc(uint32_t addr) {
  uint32_t old;
  const uint32_t one = 1u;
  asm volatile("ds_add_rtn_u32 %0, %1, %2\n\ts_waitcnt lgkmcnt(0)" : "=&v"(old) : "v"(addr), "v"(one) : "memory");
  return old;
}

// GUARD: the guard-band variant. Every tile first runs the MFMAs with the bf16 hi
// part of the query alone (half the matrix work) and forms x_hi. The entries
// whose decision x_hi >= thr the lo part could still change are those with
// |x_hi - thr| <= C ||K_s|| (Scorer::guard_c2 gives C^2; ||K_s||^2 comes from
// bf16 dot products of the key with itself, on the operands the MFMAs read).
// If any entry of the tile is that close, the wave re-reads the tile from LDS
// (this variant refills the tile's ring slots only after that) and adds the lo-part
// MFMAs to the same accumulators, which is the full computation. Otherwise
// every decision of the tile is already the full computation's. Not used when
// the sigmoid score is written: scores need the full precision everywhere.
template <int KT, int DH, int NHB, int RU, int WPB, bool GUARD>
__global__ __launch_bounds__(64 * WPB) __attribute__((amdgpu_waves_per_eu(2, 2)))
void score_stream_kernel(const ScoreArgs a) {
  static_assert(KT == KEY_BF16 || KT == KEY_FP8, "bf16 or fp8 keys");
  static_assert(RU >= 4 && RU <= 8, "ring of two to four tiles");
  constexpr int ESZ = KT == KEY_BF16 ? 2 : 1;
  constexpr int GRB = DH * ESZ;          // stored row bytes
  constexpr int UNIT = 16 * GRB;         // half tile
  static_assert(UNIT % 1024 == 0, "a half tile is whole 1 KiB load instructions");
  constexpr int NI = UNIT / 1024;        // load instructions per half tile
  constexpr int IPU = NI + (KT == KEY_FP8 ? 1 : 0);  // + the fp8 scales
  constexpr int CPR = GRB / 16;          // 16-byte chunks per row
  constexpr int NCH = CPR / 2;           // chunks of a lane's half row
  constexpr int STEPS = DH / 16;         // MFMA k-steps per head block
  // KS: a ring unit is one half of every row of a 32-row tile (bytes 0..127 or 128..255 of
  // 256-byte bf16 rows) rather than 16 whole rows, so the first half's k-steps run while the
  // second half is still landing, and each wait leaves three units in flight rather than two.
  constexpr bool KS = KT == KEY_BF16 && GRB == 256 && !GUARD;
  using S_t = Scorer<KEY_BF16, DH, NHB, false, KS>;

  __shared__ __attribute__((aligned(1024))) char rings[WPB][RU][UNIT];  // slots 1 KiB aligned
  __shared__ float srings[WPB][KT == KEY_FP8 ? RU : 1][64];
  __shared__ uint32_t next_chunk;

  const int lane = threadIdx.x & 63, g = lane >> 5, n = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  char (&ring)[RU][UNIT] = rings[wv];
  float (&sring)[KT == KEY_FP8 ? RU : 1][64] = srings[wv];
  const SeqTab t(a.key_off, a.mwo);
  const auto key_step = [](const u32x4 (&kr_)[NCH], int s_) { return key_step_t<KT, NCH>(kr_, s_); };
  if (threadIdx.x == 0) next_chunk = 0;
  __syncthreads();

  // this block's words, in chunks of CW words; the last chunk also takes the
  // remainder, so that every chunk a wave moves on to is longer than ic's
  // lead over cc (RU/2 tiles; the launcher keeps 2 CW >= RU/2 + 1) and ic
  // never claims a second chunk while cc has yet to start the first
  const int64_t nblk = gridDim.x;
  const int64_t bw0 = (int64_t)blockIdx.x * a.total_words / nblk;
  const int64_t bw1 = ((int64_t)blockIdx.x + 1) * a.total_words / nblk;
  const int64_t CW = a.chunk_words;
  const int64_t NC = max((int64_t)1, (bw1 - bw0) / CW);
#define LSA_CHUNK_WORDS(C) ((C) < NC - 1 ? CW : bw1 - bw0 - (C) * CW)
  // the next chunk of this wave (block-relative index), or -1 when all are
  // taken: one LDS increment by lane 0, read back at once
#define LSA_CLAIM(OUT)                                                                          \
  do {                                                                                          \
    uint32_t claim_v_ = 0;                                                                      \
    if (lane == 0) claim_v_ = lds_fetch_inc(lds_addr(&next_chunk));                             \
    const int64_t k_ = (int64_t)__builtin_amdgcn_readfirstlane(claim_v_);                       \
    OUT = bw1 > bw0 && k_ < NC ? k_ : -1;                                                       \
  } while (0)

  int64_t first;
  LSA_CLAIM(first);
  if (first >= 0) {
    // Per-lane offsets: the HBM chunk each lane loads for LDS position
    // k*1024 + 16*lane, and where chunk i of this lane's half row sits in LDS.
    // Both are one register XOR-ed with a constant:
    //  - load k: line 4k + lane/16, chunk lane % 16, so stream_swz(k*1024 +
    //    16*lane) = doff0 ^ (k*1024 + k*64) for k < 4 (the bit fields do not
    //    overlap);
    //  - read i: rows never cross a 256-byte line (GRB divides 256) and chunk i
    //    of the lane's half row sits at chunk-in-line p0 | i before the swizzle,
    //    so its LDS offset is roff0 ^ 16*i. Ring slots are 256-byte aligned, so
    //    the XOR also holds after the slot base is added.
    static_assert(NI <= 4 && 256 % GRB == 0, "offset identities");
    // KS: unit position P = 1024 k + 16 lane holds row 8k + lane/8 of the tile, chunk
    // (lane % 8) ^ x(row) of the row's half, with x(row) = (row / 2) % 8 (every 16 lanes of an
    // operand read then hit 16 distinct bank groups). For load k that is HBM offset
    // (8k + lane/8) * 256 + 16 ((lane % 8) ^ ((4k + lane/16) % 8)) = dks0 ^ 64 (k % 2) ^ 2048 k.
    // Lane (n, g) reads chunk 2s + g of row n (k-step s of the half) at
    // 128 n + 16 ((2s + g) ^ x(n)) = rks0 ^ 32 s.
    const uint32_t doff0 = KS ? (uint32_t)((lane >> 3) * 256 + 16 * ((lane & 7) ^ (lane >> 4))) : stream_swz(lane * 16);
    const uint32_t roff0 = KS ? (uint32_t)(n * 128 + 16 * (g ^ ((n >> 1) & 7)))
                              : stream_swz((n & 15) * GRB + 16 * (g * NCH));

    // ic: the half tiles being loaded (runs ahead); cc: the tile being scored.
    // ic always reaches the end of a chunk first; it claims the next chunk and
    // leaves its index in `pend` for cc (-1: no more work).
    WordCursor ic, cc;
    ic.place(a, t, bw0 + first * CW);
    cc = ic;
    int64_t ic_left = LSA_CHUNK_WORDS(first);  // words of the chunk, the current one included
    int64_t cc_left = ic_left;
    int64_t pend = -1;
    bool ic_live = true;
    int iq = 0;        // half tile of ic's word
    int us = 0;        // ring slot of the next half tile issued
    int cs = 0;        // ring slot of the first half of the current tile

    // Loads of the next half tile into slot us. Once ic has run out of work,
    // the half tiles get an empty buffer range: their loads fetch nothing, and
    // every iteration issues the same instructions.
#define LSA_ISSUE()                                                                               \
  do {                                                                                            \
    if constexpr (KS) {                                                                           \
      const int32_t e_ = ic.e0 + 32 * (iq >> 1);                                                  \
      const uint32_t nr_ = ic_live ? (uint32_t)uni(max(0, min(32, ic.nb - e_))) : 0u;            \
      const auto rk_ = buf_rsrc(ic.keys + (ic.row0 + e_) * GRB + 128 * (iq & 1), nr_ ? nr_ * GRB - 128 : 0u); \
      _Pragma("unroll") for (int k = 0; k < NI; ++k)                                              \
        dma_lds16(rk_, &ring[us][k * 1024], doff0 ^ (uint32_t)((k & 1) * 64 + k * 2048));         \
    } else {                                                                                      \
      const int32_t e_ = ic.e0 + 16 * iq;                                                         \
      const uint32_t nr_ = ic_live ? (uint32_t)uni(max(0, min(16, ic.nb - e_))) : 0u;            \
      const auto rk_ = buf_rsrc(ic.keys + (ic.row0 + e_) * GRB, nr_ * GRB);                       \
      _Pragma("unroll") for (int k = 0; k < NI; ++k)                                              \
        dma_lds16(rk_, &ring[us][k * 1024], doff0 ^ (uint32_t)(k * 1088));                       \
      if constexpr (KT == KEY_FP8) {                                                              \
        const auto rs_ = buf_rsrc(ic.scale + ic.row0 + e_, nr_ * 4);                              \
        dma_lds4(rs_, &sring[us][0], lane * 4);                                                  \
      }                                                                                           \
    }                                                                                             \
    us = us + 1 == RU ? 0 : us + 1;                                                               \
    if (ic_live && ++iq == 4) {                                                                   \
      iq = 0;                                                                                     \
      if (--ic_left > 0) {                                                                        \
        ic.next(a, t);                                                                            \
      } else {                                                                                    \
        int64_t nc_;                                                                              \
        LSA_CLAIM(nc_);                                                                           \
        if (nc_ >= 0) {                                                                           \
          ic.jump(a, t, bw0 + nc_ * CW);                                                          \
          ic_left = LSA_CHUNK_WORDS(nc_);                                                         \
          pend = nc_;                                                                             \
        } else {                                                                                  \
          ic_live = false;                                                                        \
          pend = -1;                                                                              \
        }                                                                                         \
      }                                                                                           \
    }                                                                                             \
  } while (0)

#pragma unroll
    for (int u = 0; u < RU; ++u) LSA_ISSUE();

    S_t S;
    int cur_l = -1, cur_b = -1;
    uint32_t bits0 = 0;
    float c2 = 0.0f;  // GUARD: C^2 of the current query
    for (int j = 0;; j ^= 1) {  // j: tile parity within the mask word
      // A new (layer, sequence)'s query, before the wait for the tile: its loads wait for every
      // load in flight (they are issued after the ring's), so the two latencies overlap.
      if (cc.l != cur_l || cc.b != cur_b) {
        S.load_query(a.q[cc.l], a.w[cc.l], cc.b, a.n_h, 0);
        if constexpr (GUARD) c2 = S.guard_c2(a.w[cc.l], cc.b, a.n_h, 0);
        cur_l = cc.l;
        cur_b = cc.b;
      }
      // the current tile is in LDS (the next RU/2 - 1 tiles may be in flight); KS: its first half
      stream_vm_wait<(RU - (KS ? 1 : 2)) * IPU>();
      const int c1 = cs + 1 == RU ? 0 : cs + 1;
      if constexpr (KS) {
        // first half of the rows: read it, refill its slot, and run its k-steps while the
        // second half lands; then the same for the second half
        f32x16 acc[NHB];
#pragma unroll
        for (int mb = 0; mb < NHB; ++mb) acc[mb] = f32x16{};
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          if (hf == 1) stream_vm_wait<(RU - 1) * IPU>();
          const uint32_t a0 = lds_addr(&ring[0][0]) + (hf ? c1 : cs) * UNIT + roff0;
          uint32_t ad[STEPS / 2];
#pragma unroll
          for (int i = 0; i < STEPS / 2; ++i) ad[i] = a0 ^ (uint32_t)(32 * i);
          u32x4 kr[STEPS / 2];
          float unused;
          lds_read_tile<STEPS / 2, false>(kr, ad, 0, unused);
          LSA_ISSUE();
#pragma unroll
          for (int s = 0; s < STEPS / 2; ++s) {
            const bf16x8 kb = as_bf16x8(kr[s]);
#pragma unroll
            for (int mb = 0; mb < NHB; ++mb) {
              acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(S.qa[mb][hf * STEPS / 2 + s][0], kb, acc[mb], 0, 0, 0);
              acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(S.qa[mb][hf * STEPS / 2 + s][1], kb, acc[mb], 0, 0, 0);
            }
          }
        }
        const float x = sum_halves(S.partial(acc));
        const int32_t se = cc.e0 + j * 32 + n;
        const bool valid = se < cc.nb;
        const uint32_t bits = (uint32_t)__ballot(valid && x >= a.thr);
        if (cc.score != nullptr && g == 0 && valid) cc.score[cc.row0 + se] = 1.0f / (1.0f + __expf(-x));
        cs = c1 + 1 == RU ? 0 : c1 + 1;
        if (j == 0) {
          bits0 = bits;
          continue;
        }
        if (lane == 0) cc.mask[cc.word] = (uint64_t)bits0 | ((uint64_t)bits << 32);
        if (--cc_left > 0) {
          cc.next(a, t);
        } else {
          if (pend < 0) break;
          cc.jump(a, t, bw0 + pend * CW);
          cc_left = LSA_CHUNK_WORDS(pend);
        }
        continue;
      }
      const int slot = n < 16 ? cs : c1;
      const uint32_t a0 = lds_addr(&ring[0][0]) + slot * UNIT + roff0;
      uint32_t ad[NCH];
#pragma unroll
      for (int i = 0; i < NCH; ++i) ad[i] = a0 ^ (uint32_t)(16 * i);
      u32x4 kr[NCH];
      float scale = 1.0f;
      lds_read_tile<NCH, KT == KEY_FP8>(kr, ad, lds_addr(&sring[0][0]) + (slot * 64 + (n & 15)) * 4, scale);
      // The reads have returned, so the tile's two ring slots are free: refill them with the tile
      // RU/2 tiles ahead now, rather than at the next iteration, so that every tile's loads are
      // in flight for RU/2 - 1 whole iterations. (The guard variant may read the tile again for
      // its lo pass, so it refills the slots after that.)
      if constexpr (!GUARD) {
        LSA_ISSUE();
        LSA_ISSUE();
      }
      f32x16 acc[NHB];
#pragma unroll
      for (int mb = 0; mb < NHB; ++mb) acc[mb] = f32x16{};
      float kn0 = 0.0f, kn1 = 0.0f;  // GUARD: this lane's share of ||K_s||^2
#pragma unroll
      for (int s = 0; s < STEPS; ++s) {
        const bf16x8 kb = key_step(kr, s);
        if constexpr (GUARD) {
          const u32x4 kd = __builtin_bit_cast(u32x4, kb);
          kn0 = dot2_bf16(kd[0], kd[0], kn0);
          kn1 = dot2_bf16(kd[1], kd[1], kn1);
          kn0 = dot2_bf16(kd[2], kd[2], kn0);
          kn1 = dot2_bf16(kd[3], kd[3], kn1);
        }
#pragma unroll
        for (int mb = 0; mb < NHB; ++mb) {
          acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(S.qa[mb][s][0], kb, acc[mb], 0, 0, 0);
          if constexpr (!GUARD) acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(S.qa[mb][s][1], kb, acc[mb], 0, 0, 0);
        }
      }
      float x = sum_halves(S.partial(acc));
      if constexpr (KT == KEY_FP8) x *= scale;
      const int32_t se = cc.e0 + j * 32 + n;
      const bool valid = se < cc.nb;
      if constexpr (GUARD) {
        // |x - x_hi| <= C ||K_s|| (times the scale for fp8). The 2^-118 floor keeps
        // the bound above the lo part's effect when the squares of a tiny key
        // underflow (every |K_i| < 2^-63 gives ||K_s|| < 2^-59).
        const float kn2 = sum_halves(kn0 + kn1) + 0x1p-118f;
        const float dlt = x - a.thr;
        float lim = c2 * kn2;
        if constexpr (KT == KEY_FP8) lim *= scale * scale;
        if (__ballot(valid && dlt * dlt <= lim) != 0) {
          u32x4 kr2[NCH];
          float unused;
          lds_read_tile<NCH, false>(kr2, ad, 0, unused);
#pragma unroll
          for (int s = 0; s < STEPS; ++s) {
            const bf16x8 kb = key_step(kr2, s);
#pragma unroll
            for (int mb = 0; mb < NHB; ++mb)
              acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(S.qa[mb][s][1], kb, acc[mb], 0, 0, 0);
          }
          x = sum_halves(S.partial(acc));
          if constexpr (KT == KEY_FP8) x *= scale;
        }
        LSA_ISSUE();
        LSA_ISSUE();
      }
      const uint32_t bits = (uint32_t)__ballot(valid && x >= a.thr);
      if (cc.score != nullptr && g == 0 && valid) cc.score[cc.row0 + se] = 1.0f / (1.0f + __expf(-x));
      cs = c1 + 1 == RU ? 0 : c1 + 1;
      if (j == 0) {
        bits0 = bits;
        continue;
      }
      if (lane == 0) cc.mask[cc.word] = (uint64_t)bits0 | ((uint64_t)bits << 32);
      if (--cc_left > 0) {
        cc.next(a, t);
      } else {
        if (pend < 0) break;
        cc.jump(a, t, bw0 + pend * CW);
        cc_left = LSA_CHUNK_WORDS(pend);
      }
    }
    // No load may still be writing this wave's LDS when it ends.
    stream_vm_wait<0>();
  }
#undef LSA_ISSUE
#undef LSA_CLAIM
#undef LSA_CHUNK_WORDS
}

constexpr int STREAM_WPB = 8;  // waves per block: two per SIMD of one CU

template <int KT, int DH, int NHB, int RU, bool GUARD>
static hipError_t launch_stream_r(const ScoreArgs& a0, int blocks, hipStream_t st) {
  // chunks must be longer than the loading cursor's lead of RU/2 tiles (two tiles per word)
  ScoreArgs a = a0;
  a.chunk_words = a.chunk_words > RU / 4 + 1 ? a.chunk_words : RU / 4 + 1;
  hipLaunchKernelGGL((score_stream_kernel<KT, DH, NHB, RU, STREAM_WPB, GUARD>), dim3(blocks), dim3(64 * STREAM_WPB), 0,
                     st, a);
  return hipGetLastError();
}

template <int KT, int DH, int NHB, int RU>
static hipError_t launch_stream_g(const ScoreArgs& a, int blocks, bool guard, hipStream_t st) {
  return guard ? launch_stream_r<KT, DH, NHB, RU, true>(a, blocks, st) : launch_stream_r<KT, DH, NHB, RU, false>(a, blocks, st);
}

template <int KT, int DH, int NHB>
static hipError_t launch_stream_h(const ScoreArgs& a, int waves, int ring, bool guard, hipStream_t st) {
  // default ring: the 8 waves of a block fit in a CU's 160 KiB of LDS
  constexpr int UNIT = 16 * DH * (KT == KEY_BF16 ? 2 : 1);
  constexpr int RDEF = UNIT >= 4096 ? 4 : 8;
  switch (ring) {
    case 4: return launch_stream_g<KT, DH, NHB, 4>(a, waves, guard, st);
    case 8: if constexpr (UNIT <= 2048) return launch_stream_g<KT, DH, NHB, 8>(a, waves, guard, st); break;
    default: break;
  }
  return launch_stream_g<KT, DH, NHB, RDEF>(a, waves, guard, st);
}

bool score_stream_supported(int key_kind, int d_h) {
  if (key_kind == KEY_BF16) return d_h == 32 || d_h == 64 || d_h == 128;
  if (key_kind == KEY_FP8) return d_h == 64 || d_h == 128;
  return false;
}

hipError_t launch_score_stream(const ScoreArgs& a, int key_kind, int d_h, int waves, int ring, bool guard,
                               hipStream_t st) {
  const bool two = a.n_h > 32;
#define LSA_STREAM_CASE(KT, DH)                                                         \
  if (key_kind == KT && d_h == DH)                                                      \
    return two ? launch_stream_h<KT, DH, 2>(a, waves, ring, guard, st) : launch_stream_h<KT, DH, 1>(a, waves, ring, guard, st);
  LSA_STREAM_CASE(KEY_BF16, 128)
  LSA_STREAM_CASE(KEY_BF16, 64)
  LSA_STREAM_CASE(KEY_BF16, 32)
  LSA_STREAM_CASE(KEY_FP8, 128)
  LSA_STREAM_CASE(KEY_FP8, 64)
#undef LSA_STREAM_CASE
  return hipErrorInvalidValue;
}

}  // namespace lsa
