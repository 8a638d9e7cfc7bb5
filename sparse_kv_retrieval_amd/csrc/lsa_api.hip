// C-ABI host layer. It validates the arguments, sizes the grids and launches
// the kernels. Every check runs before any HIP call, so a rejected call
// touches neither the device nor the stream. No allocation, no
// synchronisation.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <cstring>
#include <string>

#include "kernels.hpp"

using namespace lsa;

namespace {

thread_local std::string g_err;

lsa_status fail(lsa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

lsa_status hip_fail(const char* where, hipError_t e) {
  return fail(LSA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// Launch shapes, measured on MI355X (see the design notes): fixed at compile time.
constexpr int kScoreChunkWords = 2;    // mask words per chunk a score wave claims
constexpr int kScorePairsPerCu = 4;    // pair kernel (fp32 keys): wave pairs per CU
constexpr int kTopkPairsPerCu = 4;     // top-k scoring: wave pairs per CU
constexpr int kGatherRows = 8;         // rows per wave in flight (HBM gather)
constexpr int kFetchRows = 16;         // rows per wave in flight (host-pool fetch)
constexpr int kCopyWavesPerCu = 16;    // waves per CU of the gather and the fetch

// Checks an offsets mirror: off[0] >= 0 and non-decreasing. Also returns the total.
lsa_status check_offsets(const int64_t* off_host, int32_t B, const char* name) {
  if (!off_host) return fail(LSA_ERR_INVALID_ARG, "%s_host is NULL", name);
  if (off_host[0] < 0) return fail(LSA_ERR_INVALID_ARG, "%s_host[0] < 0", name);
  for (int32_t b = 0; b < B; ++b)
    if (off_host[b + 1] < off_host[b]) return fail(LSA_ERR_INVALID_ARG, "%s_host is decreasing at %d", name, b);
  return LSA_OK;
}

lsa_status check_seq_layout(int32_t B, const int64_t* key_offsets, const int64_t* key_offsets_host,
                            const int64_t* mwo, const int64_t* mwo_host) {
  if (B < 1) return fail(LSA_ERR_INVALID_ARG, "B must be >= 1 (got %d)", B);
  if (!key_offsets || !mwo) return fail(LSA_ERR_INVALID_ARG, "device offset array is NULL");
  lsa_status s;
  if ((s = check_offsets(key_offsets_host, B, "key_offsets")) != LSA_OK) return s;
  if ((s = check_offsets(mwo_host, B, "mask_word_offsets")) != LSA_OK) return s;
  for (int32_t b = 0; b < B; ++b) {
    const int64_t n = key_offsets_host[b + 1] - key_offsets_host[b];
    if (n > INT32_MAX) return fail(LSA_ERR_UNSUPPORTED, "sequence %d has %lld entries (> 2^31-1)", b, (long long)n);
    if (mwo_host[b + 1] - mwo_host[b] != (n + 63) / 64)
      return fail(LSA_ERR_INVALID_ARG, "mask region of sequence %d must be ceil(N_b/64) = %lld words", b,
                  (long long)((n + 63) / 64));
  }
  return LSA_OK;
}

lsa_status check_heads(int32_t n_h, int32_t d_h) {
  if (n_h < 1 || n_h > LSA_MAX_HEADS) return fail(LSA_ERR_UNSUPPORTED, "n_h must be in [1, %d] (got %d)", LSA_MAX_HEADS, n_h);
  if (d_h != 32 && d_h != 64 && d_h != 128) return fail(LSA_ERR_UNSUPPORTED, "d_h must be 32, 64 or 128 (got %d)", d_h);
  return LSA_OK;
}

// The integer a caller passed for a dtype. A C caller may pass any int, and reading a value
// that names no enumerator as the enum type would be undefined behaviour in C++, so every entry
// point takes the bits of its dtype argument first and works with the integer.
static_assert(sizeof(lsa_dtype) == sizeof(int32_t), "lsa_dtype is an int");
int32_t dtype_value(const lsa_dtype& d) {
  int32_t v;
  std::memcpy(&v, &d, sizeof v);
  return v;
}

lsa_status key_kind_of(int32_t dt, int* kind) {
  switch (dt) {
    case LSA_F32: *kind = KEY_F32; return LSA_OK;
    case LSA_BF16: *kind = KEY_BF16; return LSA_OK;
    case LSA_FP8_E4M3: *kind = KEY_FP8; return LSA_OK;
    default: return fail(LSA_ERR_UNSUPPORTED, "unknown key dtype %d", dt);
  }
}

// The kernels address one sequence's keys with 32-bit byte offsets.
lsa_status check_key_bytes(int32_t B, const int64_t* key_offsets_host, int32_t d_h, int kind) {
  const int64_t row = (int64_t)d_h * (kind == KEY_F32 ? 4 : kind == KEY_BF16 ? 2 : 1);
  for (int32_t b = 0; b < B; ++b) {
    const int64_t n = key_offsets_host[b + 1] - key_offsets_host[b];
    if (n * row > INT32_MAX)
      return fail(LSA_ERR_UNSUPPORTED, "sequence %d holds %lld bytes of keys (> 2^31-1)", b, (long long)(n * row));
  }
  return LSA_OK;
}

// The two stages of the top-k share their checks. Scoring needs the queries,
// keys and key dtype; selection needs k and the outputs; both need the lists
// and the workspace.
// contig: the layers' `keys` are the union rows packed in list order (lsa_topk_step).
lsa_status topk_stages(const lsa_topk_layer* layers, int32_t L, int32_t B, const int64_t* key_offsets,
                       const int64_t* key_offsets_host, const int32_t* idx, const int32_t* count, int32_t n_h,
                       int32_t d_h, int32_t key_dtype, int32_t k, int32_t* topk_count_out, void* workspace,
                       size_t workspace_bytes, hipStream_t stream, bool do_score, bool do_select,
                       bool contig = false) {
  if (!layers) return fail(LSA_ERR_INVALID_ARG, "layers is NULL");
  if (L < 1 || L > LSA_MAX_LAYERS) return fail(LSA_ERR_INVALID_ARG, "L must be in [1, %d] (got %d)", LSA_MAX_LAYERS, L);
  const int32_t max_b = contig ? TOPK_CONTIG_MAX_B : LSA_TOPK_MAX_B;
  if (B < 1 || B > max_b) return fail(LSA_ERR_UNSUPPORTED, "B must be in [1, %d] (got %d)", max_b, B);
  if (!key_offsets) return fail(LSA_ERR_INVALID_ARG, "key_offsets is NULL");
  lsa_status s;
  if ((s = check_offsets(key_offsets_host, B, "key_offsets")) != LSA_OK) return s;
  int kind = KEY_BF16;
  if (do_score) {
    if ((s = check_heads(n_h, d_h)) != LSA_OK) return s;
    if ((s = key_kind_of(key_dtype, &kind)) != LSA_OK) return s;
    if ((s = check_key_bytes(B, key_offsets_host, d_h, kind)) != LSA_OK) return s;
  }
  if (do_select) {
    if (k < 1 || k > 65536) return fail(LSA_ERR_UNSUPPORTED, "k must be in [1, 65536] (got %d)", k);
    if (!topk_count_out) return fail(LSA_ERR_INVALID_ARG, "topk_count_out must be set");
  }
  if (!idx || !count) return fail(LSA_ERR_INVALID_ARG, "idx and count must be set");
  const int64_t rows = key_offsets_host[B];
  for (int32_t b = 0; b < B; ++b)
    if (key_offsets_host[b + 1] - key_offsets_host[b] > INT32_MAX) return fail(LSA_ERR_UNSUPPORTED, "sequence too long");
  if (contig && rows - key_offsets_host[0] > INT32_MAX)
    return fail(LSA_ERR_UNSUPPORTED, "the packed subset rows are counted in int32 (at most 2^31-1 rows in all)");
  const size_t need = lsa_topk_workspace_size(L, B, rows, do_select ? k : 1);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(LSA_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, workspace_bytes);
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(LSA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  TopkScoreArgs sa{};
  TopkSelectArgs ta{};
  for (int l = 0; l < L; ++l) {
    const lsa_topk_layer& p = layers[l];
    if (do_score) {
      if (!p.q || !p.w || !p.keys) return fail(LSA_ERR_INVALID_ARG, "layer %d: q, w and keys must be set", l);
      if (kind == KEY_FP8 && !p.key_scale) return fail(LSA_ERR_INVALID_ARG, "layer %d: fp8 keys need key_scale", l);
      if (kind != KEY_FP8 && p.key_scale) return fail(LSA_ERR_INVALID_ARG, "layer %d: key_scale is only for fp8 keys", l);
      if (!aligned16(p.q) || !aligned16(p.keys)) return fail(LSA_ERR_INVALID_ARG, "layer %d: q and keys must be 16-byte aligned", l);
    }
    if (do_select && !p.topk_idx_out) return fail(LSA_ERR_INVALID_ARG, "layer %d: topk_idx_out must be set", l);
    sa.q[l] = p.q; sa.w[l] = p.w; sa.scale[l] = p.key_scale;
    if (contig) sa.sub_keys[l] = p.keys; else sa.keys[l] = p.keys;
    ta.out_idx[l] = p.topk_idx_out; ta.out_score[l] = p.topk_score_out;
  }
  // The scorer's histogram of each list's keys is only needed by lists too long for the select's
  // register and reload paths; a call whose sequences are all short enough skips it (and its
  // clear). The scoring and the select calls of one top-k decide the same way from the offsets.
  int64_t max_nb = 0;
  for (int32_t b = 0; b < B; ++b) max_nb = std::max<int64_t>(max_nb, key_offsets_host[b + 1] - key_offsets_host[b]);
  uint32_t* hist = max_nb > TOPK_NOHIST_MAX_ROWS ? (uint32_t*)((char*)workspace + topk_hist_offset(L, rows)) : nullptr;
  sa.ys = (float*)workspace; sa.hist = hist; sa.idx = idx; sa.count = count; sa.key_off = key_offsets;
  sa.rows_total = rows; sa.B = B; sa.L = L; sa.n_h = n_h;
  ta.ys = (const float*)workspace; ta.hist = hist; ta.idx = idx; ta.count = count; ta.key_off = key_offsets;
  ta.out_count = topk_count_out; ta.rows_total = rows; ta.B = B; ta.k = k;
  hipError_t e;
  if (do_score && hist) {
    // the histograms are counted by the scoring kernel, from zero
    if ((e = launch_topk_hist_zero(hist, (int64_t)L * B * TOPK_BINS, stream)) != hipSuccess)
      return hip_fail("lsa_topk histogram clear", e);
  }
  if (do_score && rows > 0) {
    int64_t tiles = 0;
    for (int32_t b = 0; b < B; ++b) tiles += (key_offsets_host[b + 1] - key_offsets_host[b] + 31) / 32;
    const int64_t pairs = std::max<int64_t>(1, std::min<int64_t>(tiles * L, (int64_t)cu_count() * kTopkPairsPerCu));
    if ((e = launch_topk_score(sa, kind, d_h, (int)pairs, contig, stream)) != hipSuccess)
      return hip_fail("lsa_topk score launch", e);
  }
  if (do_select && (e = launch_topk_select(ta, L, stream)) != hipSuccess) return hip_fail("lsa_topk select launch", e);
  return LSA_OK;
}

}  // namespace

extern "C" {

const char* lsa_last_error(void) { return g_err.c_str(); }

lsa_status lsa_debug_range_errors(hipStream_t stream, int64_t* count_out) {
#if LSA_DEBUG_CHECKS
  if (!count_out) return fail(LSA_ERR_INVALID_ARG, "count_out is NULL");
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail("lsa_debug_range_errors: stream", e);
  unsigned int ng = 0, nt = 0;
  if ((e = gather_take_range_errors(&ng)) != hipSuccess) return hip_fail("lsa_debug_range_errors: gather count", e);
  if ((e = topk_take_range_errors(&nt)) != hipSuccess) return hip_fail("lsa_debug_range_errors: top-k count", e);
  *count_out = (int64_t)ng + (int64_t)nt;
  return LSA_OK;
#else
  (void)stream;
  (void)count_out;
  return fail(LSA_ERR_UNSUPPORTED, "this build has no device range checks (build with LSA_DEBUG_CHECKS=1)");
#endif
}

int32_t lsa_version(void) { return LSA_VERSION; }

lsa_status lsa_project(const lsa_proj_layer* layers, int32_t L, int32_t B, int32_t d, int32_t r, int32_t n_h,
                       int32_t d_h, lsa_dtype dtype_arg, hipStream_t stream) {
  const int32_t dtype = dtype_value(dtype_arg);
  if (!layers) return fail(LSA_ERR_INVALID_ARG, "layers is NULL");
  if (L < 1 || L > LSA_MAX_LAYERS) return fail(LSA_ERR_INVALID_ARG, "L must be in [1, %d] (got %d)", LSA_MAX_LAYERS, L);
  if (B < 1 || B > 128) return fail(LSA_ERR_UNSUPPORTED, "B must be in [1, 128] (got %d)", B);
  if (dtype != LSA_F32 && dtype != LSA_BF16) return fail(LSA_ERR_UNSUPPORTED, "projection dtype must be LSA_F32 or LSA_BF16");
  const int kq = dtype == LSA_F32 ? 4 : 32;
  if (d < kq || d % kq || r < kq || r % kq)
    return fail(LSA_ERR_UNSUPPORTED, "d and r must be positive multiples of %d (got d=%d r=%d)", kq, d, r);
  if (n_h < 1 || n_h > LSA_MAX_HEADS || d_h < 1) return fail(LSA_ERR_UNSUPPORTED, "bad head shape n_h=%d d_h=%d", n_h, d_h);
  if ((int64_t)n_h * d_h % 16) return fail(LSA_ERR_UNSUPPORTED, "n_h*d_h must be a multiple of 16");
  ProjArgs a{};
  for (int l = 0; l < L; ++l) {
    const lsa_proj_layer& p = layers[l];
    if (!p.h || !p.w_dq || !p.w_iuq || !p.w_w || !p.c_out || !p.q_out || !p.w_out)
      return fail(LSA_ERR_INVALID_ARG, "layer %d: a pointer is NULL", l);
    if (!aligned16(p.h) || !aligned16(p.w_dq) || !aligned16(p.w_iuq) || !aligned16(p.w_w) || !aligned16(p.c_out))
      return fail(LSA_ERR_INVALID_ARG, "layer %d: h, w_dq, w_iuq, w_w and c_out must be 16-byte aligned", l);
    if ((const void*)p.c_out == (const void*)p.q_out || (const void*)p.c_out == (const void*)p.w_out)
      return fail(LSA_ERR_INVALID_ARG, "layer %d: c_out aliases another output", l);
    a.h[l] = p.h; a.w_dq[l] = p.w_dq; a.w_iuq[l] = p.w_iuq; a.w_w[l] = p.w_w;
    a.c[l] = p.c_out; a.q[l] = p.q_out; a.w[l] = p.w_out;
  }
  a.B = B; a.d = d; a.r = r; a.n_h = n_h; a.d_h = d_h;
  const hipError_t e = launch_project(a, L, dtype == LSA_F32, stream);
  return e == hipSuccess ? LSA_OK : hip_fail("lsa_project launch", e);
}

size_t lsa_pack_weights_size(int32_t rows, int32_t K) {
  if (rows < 1 || K < 32 || K % 32) return 0;
  return (size_t)((rows + 15) / 16) * (size_t)(K / 32) * 1024;
}

lsa_status lsa_pack_weights(const void* w, int32_t rows, int32_t K, void* out, size_t out_bytes, hipStream_t stream) {
  if (!w || !out) return fail(LSA_ERR_INVALID_ARG, "w and out must be set");
  if (rows < 1 || K < 32 || K % 32) return fail(LSA_ERR_UNSUPPORTED, "rows >= 1 and K a positive multiple of 32 (got %d x %d)", rows, K);
  if (!aligned16(w) || !aligned16(out)) return fail(LSA_ERR_INVALID_ARG, "w and out must be 16-byte aligned");
  const size_t need = lsa_pack_weights_size(rows, K);
  if (need > (size_t)INT32_MAX) return fail(LSA_ERR_UNSUPPORTED, "packed matrix of %zu bytes (> 2^31-1)", need);
  if (out_bytes < need) return fail(LSA_ERR_INVALID_ARG, "out holds %zu bytes, packing needs %zu", out_bytes, need);
  const hipError_t e = launch_pack_weights(w, rows, K, out, stream);
  return e == hipSuccess ? LSA_OK : hip_fail("lsa_pack_weights launch", e);
}

lsa_status lsa_project_packed(const lsa_proj_layer* layers, int32_t L, int32_t B, int32_t d, int32_t r, int32_t n_h,
                              int32_t d_h, hipStream_t stream) {
  if (!layers) return fail(LSA_ERR_INVALID_ARG, "layers is NULL");
  if (L < 1 || L > LSA_MAX_LAYERS) return fail(LSA_ERR_INVALID_ARG, "L must be in [1, %d] (got %d)", LSA_MAX_LAYERS, L);
  if (B < 1 || B > 32) return fail(LSA_ERR_UNSUPPORTED, "B must be in [1, 32] for packed weights (got %d)", B);
  if (d < 32 || d % 32 || r < 64 || r % 64)
    return fail(LSA_ERR_UNSUPPORTED, "d must be a positive multiple of 32 and r of 64 (got d=%d r=%d)", d, r);
  if (n_h < 1 || n_h > LSA_MAX_HEADS || d_h < 1) return fail(LSA_ERR_UNSUPPORTED, "bad head shape n_h=%d d_h=%d", n_h, d_h);
  if ((int64_t)n_h * d_h % 64) return fail(LSA_ERR_UNSUPPORTED, "n_h*d_h must be a multiple of 64");
  if (lsa_pack_weights_size(n_h * d_h, r) > (size_t)INT32_MAX || lsa_pack_weights_size(r, d) > (size_t)INT32_MAX ||
      (int64_t)B * d * 2 > INT32_MAX || (int64_t)B * r * 4 > INT32_MAX)
    return fail(LSA_ERR_UNSUPPORTED, "a packed matrix or an activation exceeds 2^31-1 bytes");
  ProjArgs a{};
  for (int l = 0; l < L; ++l) {
    const lsa_proj_layer& p = layers[l];
    if (!p.h || !p.w_dq || !p.w_iuq || !p.w_w || !p.c_out || !p.q_out || !p.w_out)
      return fail(LSA_ERR_INVALID_ARG, "layer %d: a pointer is NULL", l);
    if (!aligned16(p.h) || !aligned16(p.w_dq) || !aligned16(p.w_iuq) || !aligned16(p.w_w) || !aligned16(p.c_out))
      return fail(LSA_ERR_INVALID_ARG, "layer %d: h, the packed weights and c_out must be 16-byte aligned", l);
    if ((const void*)p.c_out == (const void*)p.q_out || (const void*)p.c_out == (const void*)p.w_out)
      return fail(LSA_ERR_INVALID_ARG, "layer %d: c_out aliases another output", l);
    a.h[l] = p.h; a.w_dq[l] = p.w_dq; a.w_iuq[l] = p.w_iuq; a.w_w[l] = p.w_w;
    a.c[l] = p.c_out; a.q[l] = p.q_out; a.w[l] = p.w_out;
  }
  a.B = B; a.d = d; a.r = r; a.n_h = n_h; a.d_h = d_h;
  const hipError_t e = launch_project_packed(a, L, stream);
  return e == hipSuccess ? LSA_OK : hip_fail("lsa_project_packed launch", e);
}

}  // extern "C"

namespace {
lsa_status score_select_impl(const lsa_score_layer* layers, int32_t L, int32_t B, const int64_t* key_offsets,
                             const int64_t* key_offsets_host, const int64_t* mask_word_offsets,
                             const int64_t* mask_word_offsets_host, int32_t n_h, int32_t d_h, int32_t key_dtype,
                             float threshold, const lsa_score_options* options, hipStream_t stream) {
  if (!layers) return fail(LSA_ERR_INVALID_ARG, "layers is NULL");
  if (L < 1 || L > LSA_MAX_LAYERS) return fail(LSA_ERR_INVALID_ARG, "L must be in [1, %d] (got %d)", LSA_MAX_LAYERS, L);
  lsa_status s;
  if ((s = check_seq_layout(B, key_offsets, key_offsets_host, mask_word_offsets, mask_word_offsets_host)) != LSA_OK) return s;
  if ((s = check_heads(n_h, d_h)) != LSA_OK) return s;
  int kind;
  if ((s = key_kind_of(key_dtype, &kind)) != LSA_OK) return s;
  if ((s = check_key_bytes(B, key_offsets_host, d_h, kind)) != LSA_OK) return s;
  if (!(threshold > 0.0f && threshold < 1.0f)) return fail(LSA_ERR_INVALID_ARG, "threshold must lie in (0, 1)");
  lsa_score_options opt{LSA_SCORE_KERNEL_AUTO, 0, 0, 0};
  if (options) {
    opt = *options;
    if (opt.kernel < LSA_SCORE_KERNEL_AUTO || opt.kernel > LSA_SCORE_KERNEL_PAIRS)
      return fail(LSA_ERR_INVALID_ARG, "options->kernel must be 0, 1 or 2 (got %d)", opt.kernel);
    if (opt.chunk_words != 0 && (opt.chunk_words < 2 || opt.chunk_words > 64))
      return fail(LSA_ERR_INVALID_ARG, "options->chunk_words must be 0 or in [2, 64] (got %d)", opt.chunk_words);
    if (opt.ring != 0 && opt.ring != 4 && opt.ring != 8)
      return fail(LSA_ERR_INVALID_ARG, "options->ring must be 0, 4 or 8 (got %d)", opt.ring);
    if (opt.guard != 0 && opt.guard != 1) return fail(LSA_ERR_INVALID_ARG, "options->guard must be 0 or 1");
  }
  const bool stream_ok = score_stream_supported(kind, d_h);
  if (opt.kernel == LSA_SCORE_KERNEL_STREAM && !stream_ok)
    return fail(LSA_ERR_UNSUPPORTED, "the one-wave-per-tile kernel takes bf16 keys (d_h 32, 64, 128) or fp8 keys (d_h 64, 128)");
  ScoreArgs a{};
  bool scores = false;
  for (int l = 0; l < L; ++l) {
    const lsa_score_layer& p = layers[l];
    if (!p.q || !p.w || !p.keys || !p.mask_out) return fail(LSA_ERR_INVALID_ARG, "layer %d: q, w, keys and mask_out must be set", l);
    if (kind == KEY_FP8 && !p.key_scale) return fail(LSA_ERR_INVALID_ARG, "layer %d: fp8 keys need key_scale", l);
    if (kind != KEY_FP8 && p.key_scale) return fail(LSA_ERR_INVALID_ARG, "layer %d: key_scale is only for fp8 keys", l);
    if (!aligned16(p.q) || !aligned16(p.keys)) return fail(LSA_ERR_INVALID_ARG, "layer %d: q and keys must be 16-byte aligned", l);
    a.q[l] = p.q; a.w[l] = p.w; a.keys[l] = p.keys; a.scale[l] = p.key_scale;
    a.mask[l] = p.mask_out; a.score[l] = p.score_out;
    scores |= p.score_out != nullptr;
  }
  const double t = std::log((double)threshold / (1.0 - (double)threshold));
  a.key_off = key_offsets; a.mwo = mask_word_offsets;
  a.word_base = mask_word_offsets_host[0];
  a.words_per_layer = mask_word_offsets_host[B] - mask_word_offsets_host[0];
  a.total_words = a.words_per_layer * L;
  a.B = B; a.n_h = n_h; a.L = L; a.thr = (float)t;
  if (a.total_words == 0) return LSA_OK;
  if (stream_ok && opt.kernel != LSA_SCORE_KERNEL_PAIRS) {
    // one block of 8 waves per CU, each block a contiguous run of mask words
    // that its waves take in chunks of a few words
    a.chunk_words = opt.chunk_words ? opt.chunk_words : kScoreChunkWords;
    const int64_t waves = std::min<int64_t>((a.total_words + 7) / 8, (int64_t)cu_count());
    a.group = 1;
    // the hi-only first pass decides masks only; the sigmoid scores need the full pass everywhere
    const bool guard = !scores && opt.guard;
    const hipError_t e = launch_score_stream(a, kind, d_h, (int)waves, opt.ring, guard, stream);
    return e == hipSuccess ? LSA_OK : hip_fail("lsa_score_select launch", e);
  }
  // One block per pair of waves over a contiguous run of words.
  const int64_t pairs = std::min<int64_t>(a.total_words, (int64_t)cu_count() * kScorePairsPerCu);
  a.group = 1;
  const hipError_t e = launch_score_select(a, kind, d_h, (int)pairs, 0, stream);
  return e == hipSuccess ? LSA_OK : hip_fail("lsa_score_select launch", e);
}

}  // namespace

extern "C" {

lsa_status lsa_score_select_ex(const lsa_score_layer* layers, int32_t L, int32_t B, const int64_t* key_offsets,
                               const int64_t* key_offsets_host, const int64_t* mask_word_offsets,
                               const int64_t* mask_word_offsets_host, int32_t n_h, int32_t d_h, lsa_dtype key_dtype,
                               float threshold, const lsa_score_options* options, hipStream_t stream) {
  return score_select_impl(layers, L, B, key_offsets, key_offsets_host, mask_word_offsets, mask_word_offsets_host,
                           n_h, d_h, dtype_value(key_dtype), threshold, options, stream);
}

lsa_status lsa_score_select(const lsa_score_layer* layers, int32_t L, int32_t B, const int64_t* key_offsets,
                            const int64_t* key_offsets_host, const int64_t* mask_word_offsets,
                            const int64_t* mask_word_offsets_host, int32_t n_h, int32_t d_h, lsa_dtype key_dtype,
                            float threshold, hipStream_t stream) {
  return score_select_impl(layers, L, B, key_offsets, key_offsets_host, mask_word_offsets, mask_word_offsets_host,
                           n_h, d_h, dtype_value(key_dtype), threshold, nullptr, stream);
}

lsa_status lsa_union_compact(const uint64_t* const* masks, int32_t L, int32_t B, const int64_t* key_offsets,
                             const int64_t* key_offsets_host, const int64_t* mask_word_offsets,
                             const int64_t* mask_word_offsets_host, int32_t* idx_out, int32_t* count_out,
                             uint64_t* union_mask_out, hipStream_t stream) {
  if (!masks) return fail(LSA_ERR_INVALID_ARG, "masks is NULL");
  if (L < 1 || L > LSA_MAX_LAYERS) return fail(LSA_ERR_INVALID_ARG, "L must be in [1, %d] (got %d)", LSA_MAX_LAYERS, L);
  if (B > 65535) return fail(LSA_ERR_UNSUPPORTED, "B must be <= 65535");
  lsa_status s;
  if ((s = check_seq_layout(B, key_offsets, key_offsets_host, mask_word_offsets, mask_word_offsets_host)) != LSA_OK) return s;
  if (!idx_out || !count_out) return fail(LSA_ERR_INVALID_ARG, "idx_out and count_out must be set");
  UnionArgs a{};
  for (int l = 0; l < L; ++l) {
    if (!masks[l]) return fail(LSA_ERR_INVALID_ARG, "masks[%d] is NULL", l);
    a.mask[l] = masks[l];
  }
  int64_t max_words = 0;
  for (int b = 0; b < B; ++b) max_words = std::max(max_words, mask_word_offsets_host[b + 1] - mask_word_offsets_host[b]);
  a.key_off = key_offsets; a.mwo = mask_word_offsets; a.idx_out = idx_out; a.count_out = count_out;
  a.union_out = union_mask_out; a.L = L;
  const hipError_t e = launch_union_compact(a, B, max_words, cu_count(), stream);
  return e == hipSuccess ? LSA_OK : hip_fail("lsa_union_compact launch", e);
}

size_t lsa_topk_workspace_size(int32_t L, int32_t B, int64_t total_rows, int32_t k) {
  (void)k;
  if (L < 1 || B < 1 || total_rows < 0) return 0;
  return topk_workspace_bytes(L, B, total_rows);
}

lsa_status lsa_topk(const lsa_topk_layer* layers, int32_t L, int32_t B, const int64_t* key_offsets,
                    const int64_t* key_offsets_host, const int32_t* idx, const int32_t* count, int32_t n_h, int32_t d_h,
                    lsa_dtype key_dtype, int32_t k, int32_t* topk_count_out, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
  return topk_stages(layers, L, B, key_offsets, key_offsets_host, idx, count, n_h, d_h, dtype_value(key_dtype), k,
                     topk_count_out, workspace, workspace_bytes, stream, true, true);
}

lsa_status lsa_topk_score(const lsa_topk_layer* layers, int32_t L, int32_t B, const int64_t* key_offsets,
                          const int64_t* key_offsets_host, const int32_t* idx, const int32_t* count, int32_t n_h,
                          int32_t d_h, lsa_dtype key_dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return topk_stages(layers, L, B, key_offsets, key_offsets_host, idx, count, n_h, d_h, dtype_value(key_dtype), 1,
                     nullptr, workspace, workspace_bytes, stream, true, false);
}

lsa_status lsa_topk_step(const lsa_topk_layer* layers, int32_t L, int32_t B, const int64_t* key_offsets,
                         const int64_t* key_offsets_host, const int32_t* idx, const int32_t* count, int32_t n_h,
                         int32_t d_h, lsa_dtype key_dtype, int32_t k, int32_t* topk_count_out, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  return topk_stages(layers, L, B, key_offsets, key_offsets_host, idx, count, n_h, d_h, dtype_value(key_dtype), k,
                     topk_count_out, workspace, workspace_bytes, stream, true, true, true);
}

}  // extern "C"

// Scratch of lsa_topk_step_noalloc: a fixed array in device memory, one copy on
// every GPU the library runs on, held until the process ends. Host code never
// passes the array's name to a kernel (on the host it is only a stand-in); it
// takes the device's address of its copy from hipGetSymbolAddress, once per
// device, and passes that.
static __device__ __align__(256) char scratch[LSA_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {nullptr};

// The current device's address of `scratch` (looked up on the first call on that device).
lsa_status scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail("lsa_topk_step_noalloc: hipGetDevice", e);
  if (dev < 0 || dev >= 64) return fail(LSA_ERR_UNSUPPORTED, "lsa_topk_step_noalloc: device %d (at most 64)", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return hip_fail("lsa_topk_step_noalloc: hipGetSymbolAddress", e);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return LSA_OK;
}
}  // namespace

extern "C" {

lsa_status lsa_topk_step_noalloc(const lsa_topk_layer* layers, int32_t L, int32_t B, const int64_t* key_offsets,
                                 const int64_t* key_offsets_host, const int32_t* idx, const int32_t* count,
                                 int32_t n_h, int32_t d_h, lsa_dtype key_dtype, int32_t k, int32_t* topk_count_out,
                                 hipStream_t stream) {
  // the size check needs only host values, and runs before any HIP call
  if (L < 1 || L > LSA_MAX_LAYERS) return fail(LSA_ERR_INVALID_ARG, "L must be in [1, %d] (got %d)", LSA_MAX_LAYERS, L);
  if (B < 1 || B > TOPK_CONTIG_MAX_B) return fail(LSA_ERR_UNSUPPORTED, "B must be in [1, %d] (got %d)", TOPK_CONTIG_MAX_B, B);
  lsa_status s;
  if ((s = check_offsets(key_offsets_host, B, "key_offsets")) != LSA_OK) return s;
  const size_t need = lsa_topk_workspace_size(L, B, key_offsets_host[B], k);
  if (need > (size_t)LSA_NOALLOC_SCRATCH_BYTES)
    return fail(LSA_ERR_UNSUPPORTED, "lsa_topk_step_noalloc: the call needs %zu bytes of scratch, more than the %d the "
                                     "library holds (use lsa_topk_step with a workspace)", need, LSA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((s = scratch_for_current_device(&ws)) != LSA_OK) return s;
  return topk_stages(layers, L, B, key_offsets, key_offsets_host, idx, count, n_h, d_h, dtype_value(key_dtype), k,
                     topk_count_out, ws, (size_t)LSA_NOALLOC_SCRATCH_BYTES, stream, true, true, true);
}

lsa_status lsa_topk_select(const lsa_topk_layer* layers, int32_t L, int32_t B, const int64_t* key_offsets,
                           const int64_t* key_offsets_host, const int32_t* idx, const int32_t* count, int32_t k,
                           int32_t* topk_count_out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return topk_stages(layers, L, B, key_offsets, key_offsets_host, idx, count, 1, 32, LSA_BF16, k, topk_count_out,
                     workspace, workspace_bytes, stream, false, true);
}

}  // extern "C"

namespace {
// Argument checks and launch shared by lsa_gather and lsa_fetch_host; `pool`
// is the address the kernel reads through.
lsa_status gather_call(const char* what, const void* pool, int64_t row_bytes, int32_t B,
                       const int64_t* pool_row_offsets, const int64_t* pool_row_offsets_host, const int32_t* idx,
                       const int64_t* idx_offsets, const int32_t* count, void* out, const int64_t* out_row_offsets,
                       int64_t out_capacity_rows, int rows_per_wave, int waves_per_cu, hipStream_t stream) {
  if (B < 1 || B > LSA_TOPK_MAX_B) return fail(LSA_ERR_UNSUPPORTED, "B must be in [1, %d] (got %d)", LSA_TOPK_MAX_B, B);
  if (row_bytes <= 0 || row_bytes % 16) return fail(LSA_ERR_INVALID_ARG, "row_bytes must be a positive multiple of 16");
  if (!pool || !pool_row_offsets || !idx || !idx_offsets || !count || !out)
    return fail(LSA_ERR_INVALID_ARG, "pool, pool_row_offsets, idx, idx_offsets, count and out must be set");
  if (!aligned16(pool) || !aligned16(out)) return fail(LSA_ERR_INVALID_ARG, "pool and out must be 16-byte aligned");
  if (out_capacity_rows < 0) return fail(LSA_ERR_INVALID_ARG, "out_capacity_rows < 0");
  lsa_status s;
  if ((s = check_offsets(pool_row_offsets_host, B, "pool_row_offsets")) != LSA_OK) return s;
  const int64_t bound = std::min<int64_t>(out_capacity_rows, pool_row_offsets_host[B] - pool_row_offsets_host[0]);
  if (bound == 0) {
    // Nothing can be written, but the call is still well formed.
    return LSA_OK;
  }
  GatherArgs a{};
  a.pool = (const char*)pool; a.pool_off = pool_row_offsets; a.idx = idx; a.idx_off = idx_offsets; a.count = count;
  a.out = (char*)out; a.out_off = out_row_offsets; a.out_capacity = out_capacity_rows; a.row_bytes = row_bytes; a.B = B;
  const int64_t waves = std::min<int64_t>((bound + rows_per_wave - 1) / rows_per_wave, (int64_t)cu_count() * waves_per_cu);
  const hipError_t e = launch_gather(a, (int)((waves + 3) / 4), rows_per_wave, stream);
  return e == hipSuccess ? LSA_OK : hip_fail(what, e);
}
}  // namespace

extern "C" {

lsa_status lsa_gather(const void* pool, int64_t row_bytes, int32_t B, const int64_t* pool_row_offsets,
                      const int64_t* pool_row_offsets_host, const int32_t* idx, const int64_t* idx_offsets,
                      const int32_t* count, void* out, const int64_t* out_row_offsets, int64_t out_capacity_rows,
                      hipStream_t stream) {
  return gather_call("lsa_gather launch", pool, row_bytes, B, pool_row_offsets, pool_row_offsets_host, idx, idx_offsets,
                     count, out, out_row_offsets, out_capacity_rows, kGatherRows, kCopyWavesPerCu, stream);
}

lsa_status lsa_fetch_host(const void* pool_host, int64_t row_bytes, int32_t B, const int64_t* pool_row_offsets,
                          const int64_t* pool_row_offsets_host, const int32_t* idx, const int64_t* idx_offsets,
                          const int32_t* count, void* out, const int64_t* out_row_offsets, int64_t out_capacity_rows,
                          hipStream_t stream) {
  if (!pool_host) return fail(LSA_ERR_INVALID_ARG, "pool_host is NULL");
  // The pool must be pinned host memory that the device can read (hipHostMalloc).
  hipPointerAttribute_t attr{};
  const hipError_t pe = hipPointerGetAttributes(&attr, pool_host);
  if (pe != hipSuccess || attr.type != hipMemoryTypeHost || attr.devicePointer == nullptr) {
    (void)hipGetLastError();  // leave no error behind for the caller's next HIP call
    return fail(LSA_ERR_INVALID_ARG, "pool_host must be pinned host memory allocated with hipHostMalloc");
  }
  // the device's address for pool_host (the attributes may describe the whole allocation)
  const char* dev_view = attr.hostPointer
                             ? (const char*)attr.devicePointer + ((const char*)pool_host - (const char*)attr.hostPointer)
                             : (const char*)attr.devicePointer;
  return gather_call("lsa_fetch_host launch", dev_view, row_bytes, B, pool_row_offsets, pool_row_offsets_host, idx,
                     idx_offsets, count, out, out_row_offsets, out_capacity_rows, kFetchRows, kCopyWavesPerCu, stream);
}

size_t lsa_golden_workspace_size(int32_t T, int32_t L, int64_t row_stride) {
  if (T < 1 || L < 1 || row_stride < 1) return 0;
  return golden_workspace_bytes((int64_t)T * L, row_stride);
}

lsa_status lsa_golden_labels(const float* logits, int64_t row_stride, int32_t T, int32_t L, const int32_t* n_valid,
                             float top_p, int32_t theta, uint64_t* row_mask_out, int32_t* nucleus_size_out,
                             uint64_t* token_golden_out, uint64_t* golden_out, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  if (!logits || !n_valid || !row_mask_out || !golden_out)
    return fail(LSA_ERR_INVALID_ARG, "logits, n_valid, row_mask_out and golden_out must be set");
  if (T < 1 || L < 1 || L > 64) return fail(LSA_ERR_INVALID_ARG, "need T >= 1 and 1 <= L <= 64 (got T=%d L=%d)", T, L);
  if ((int64_t)T * L > INT32_MAX) return fail(LSA_ERR_UNSUPPORTED, "T * L must fit in int32");
  if (row_stride < 1 || row_stride > LSA_GOLDEN_MAX_ROW)
    return fail(LSA_ERR_UNSUPPORTED, "row_stride must be in [1, %d] (got %lld)", LSA_GOLDEN_MAX_ROW,
                (long long)row_stride);
  if (!(top_p > 0.0f && top_p <= 1.0f)) return fail(LSA_ERR_INVALID_ARG, "top_p must be in (0, 1]");
  if (theta < 1) return fail(LSA_ERR_INVALID_ARG, "theta must be >= 1 (got %d)", theta);
  if ((reinterpret_cast<uintptr_t>(logits) & 3u) || (reinterpret_cast<uintptr_t>(row_mask_out) & 7u) ||
      (reinterpret_cast<uintptr_t>(golden_out) & 7u) || (reinterpret_cast<uintptr_t>(token_golden_out) & 7u))
    return fail(LSA_ERR_INVALID_ARG, "logits must be 4-byte and mask buffers 8-byte aligned");
  const size_t need = golden_workspace_bytes((int64_t)T * L, row_stride);
  if (!workspace || workspace_bytes < need)
    return fail(LSA_ERR_WORKSPACE, "lsa_golden_labels needs a workspace of %zu bytes (got %zu)", need, workspace_bytes);
  if (reinterpret_cast<uintptr_t>(workspace) & 15u) return fail(LSA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  GoldenArgs a{};
  a.ws = (char*)workspace;
  a.logits = logits; a.n_valid = n_valid; a.row_mask = row_mask_out; a.nucleus_size = nucleus_size_out;
  a.token_golden = token_golden_out; a.golden = golden_out;
  a.row_stride = row_stride; a.W = (row_stride + 63) / 64; a.T = T; a.L = L; a.p = top_p;
  a.theta = theta > 127 ? 127 : theta;  // more votes than layers: nothing is golden either way
  const hipError_t e = launch_golden(a, stream);
  return e == hipSuccess ? LSA_OK : hip_fail("lsa_golden_labels launch", e);
}

size_t lsa_train_workspace_size(int32_t B, const int64_t* key_offsets_host, int32_t r) {
  if (B < 1 || !key_offsets_host || r < 1) return 0;
  return train_workspace_bytes(B, r, train_scan_blocks(key_offsets_host, B, nullptr));
}

lsa_status lsa_train_step(const void* h, const void* w_dq, const void* w_iuq, const void* w_w, const void* keys,
                          const int64_t* key_offsets, const int64_t* key_offsets_host, const uint64_t* labels,
                          const int64_t* mask_word_offsets, const int64_t* mask_word_offsets_host, int32_t B,
                          int32_t d, int32_t r, int32_t n_h, int32_t d_h, float gamma, float alpha, float* loss_out,
                          float* g_dq, float* g_iuq, float* g_w, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  if (!h || !w_dq || !w_iuq || !w_w || !keys || !labels || !loss_out || !g_dq || !g_iuq || !g_w)
    return fail(LSA_ERR_INVALID_ARG, "h, the weights, keys, labels, loss_out and the gradients must be set");
  if (B < 1 || B > 32) return fail(LSA_ERR_UNSUPPORTED, "B must be in [1, 32] (got %d)", B);
  if (n_h != 64 || d_h != 128) return fail(LSA_ERR_UNSUPPORTED, "the training step needs n_h = 64, d_h = 128");
  if (d < 32 || d % 32 || r < 32 || r % 32)
    return fail(LSA_ERR_UNSUPPORTED, "d and r must be positive multiples of 32 (got d=%d r=%d)", d, r);
  if (!(gamma >= 0.f && gamma < 1e6f) || !(alpha >= 0.f && alpha <= 1.f))
    return fail(LSA_ERR_INVALID_ARG, "need gamma >= 0 and 0 <= alpha <= 1");
  lsa_status s;
  if ((s = check_seq_layout(B, key_offsets, key_offsets_host, mask_word_offsets, mask_word_offsets_host)) != LSA_OK)
    return s;
  for (int32_t b = 0; b < B; ++b)
    if ((key_offsets_host[b + 1] - key_offsets_host[b]) * 256 >= ((int64_t)1 << 31))
      return fail(LSA_ERR_UNSUPPORTED, "sequence %d is longer than the training scan addresses (2^23 entries)", b);
  if (!aligned16(h) || !aligned16(w_dq) || !aligned16(w_iuq) || !aligned16(w_w) || !aligned16(keys) ||
      !aligned16(workspace))
    return fail(LSA_ERR_INVALID_ARG, "h, w_dq, w_iuq, w_w, keys and workspace must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(labels) & 7u) || (reinterpret_cast<uintptr_t>(g_dq) & 15u) ||
      (reinterpret_cast<uintptr_t>(g_iuq) & 15u) || (reinterpret_cast<uintptr_t>(g_w) & 15u) ||
      (reinterpret_cast<uintptr_t>(loss_out) & 3u))
    return fail(LSA_ERR_INVALID_ARG, "labels must be 8-byte aligned, the gradients 16-byte and loss_out 4-byte aligned");
  int tpb = 0;
  const int64_t nblk = train_scan_blocks(key_offsets_host, B, &tpb);
  const size_t need = train_workspace_bytes(B, r, nblk);
  if (!workspace || workspace_bytes < need)
    return fail(LSA_ERR_WORKSPACE, "lsa_train_step needs a workspace of %zu bytes (got %zu)", need, workspace_bytes);
  const int64_t total = key_offsets_host[B] - key_offsets_host[0];
  const TrainWs ws = train_carve(workspace, B, r, nblk);
  ProjArgs p{};
  p.h[0] = h; p.w_dq[0] = w_dq; p.w_iuq[0] = w_iuq; p.w_w[0] = w_w;
  p.c[0] = ws.c; p.q[0] = ws.q; p.w[0] = ws.w;
  p.B = B; p.d = d; p.r = r; p.n_h = n_h; p.d_h = d_h;
  // c, q, w are contiguous in the workspace; the split projection adds into them
  hipError_t e = launch_train_zero(ws.c, (int64_t)B * (r + n_h * d_h + n_h), stream);
  if (e == hipSuccess) e = launch_project_split2(p, stream);
  if (e != hipSuccess) return hip_fail("lsa_train_step projection", e);
  TrainArgs a{};
  a.keys = keys; a.key_off = key_offsets; a.labels = labels; a.mwo = mask_word_offsets; a.h = h; a.w_iuq = w_iuq;
  a.c = ws.c; a.q = ws.q; a.w = ws.w; a.part = ws.part; a.dq = ws.dq; a.dw = ws.dw; a.dc = ws.dc; a.dcp = ws.dcp;
  a.loss = loss_out;
  a.g_dq = g_dq; a.g_iuq = g_iuq; a.g_w = g_w; a.nblk = nblk; a.tpb = tpb; a.B = B; a.d = d; a.r = r;
  a.gamma = gamma; a.alpha = alpha; a.inv_total = total > 0 ? (float)(1.0 / (double)total) : 0.f;
  e = launch_train(a, stream);
  return e == hipSuccess ? LSA_OK : hip_fail("lsa_train_step launch", e);
}

}  // extern "C"
