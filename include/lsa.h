/*
 * lsa.h: C-ABI of the MI355X (gfx950) LSA memory-indexer selection path.
 *
 * The library implements one trigger of the Lookahead Sparse Attention memory
 * indexer. The method is described in the write-up "arXiv'26 |
 * FlashMemory-DeepSeek-V4: 用 13.5% 的显存干 100% 的活, 超长上下文推理的 less is
 * more" (marsggbo.github.io, cited below as [BLOG]) and in the hyper.ai digest
 * of the same report (section "方法", cited as [HYPER]). The steps are:
 *
 *   lsa_project        c = h W^DQ, q = c W^IUQ, w = h W^w        [BLOG] §3.1
 *   (lsa_project_packed, the same with weights packed once by lsa_pack_weights)
 *   lsa_score_select   I_s = sigma(sum_j w_j ReLU(q_j . K_s)), keep I_s >= theta
 *                                                                [BLOG] §3.1
 *   lsa_union_compact  OR over the indexer layers, ascending index list
 *                                                    [BLOG] §4.2, [HYPER] 方法
 *   lsa_topk           native Lightning-Indexer top-k inside the subset
 *                                                    [BLOG] §2.2, §3.2
 *   lsa_topk_step      the same at every decode step, over the subset's keys
 *                      packed once per trigger              [BLOG] §3.2
 *   lsa_gather         copy the selected compressed-KV rows into a compact buffer
 *                                                    [HYPER] 方法 (load C^MemComp)
 *   lsa_fetch_host     the same copy from a pool in pinned host memory
 *                                                    [HYPER] 方法, [BLOG] §3
 *   lsa_golden_labels  training targets: per-layer softmax top-p nucleus,
 *                      cross-layer vote, union over the lookahead window
 *                                                    [HYPER] 数据集, [BLOG] §4.1
 *   lsa_train_step     one training step of an indexer layer: focal BCE of
 *                      the score against golden labels, gradients of W^DQ,
 *                      W^IUQ and W^w with the keys frozen
 *                                                  [BLOG] §4 训练, [HYPER] 方法
 *
 * Conventions shared by every call:
 *  - Ownership: the caller allocates every buffer. Pointers marked "dev" are
 *    device memory on the current HIP device; pointers marked "host" are host
 *    memory read during the call only. The library never allocates, frees or
 *    synchronises. Its only scratch space is the caller's workspace (top-k,
 *    golden labels and the training step).
 *  - Asynchrony: kernels are enqueued on `stream` and the call returns at once.
 *    Results are valid once the stream reaches that point. Calls are reentrant.
 *  - Errors: every argument is checked on the host before anything is enqueued.
 *    A bad argument returns LSA_ERR_INVALID_ARG and an unsupported shape or
 *    dtype returns LSA_ERR_UNSUPPORTED. In both cases nothing is launched and
 *    lsa_last_error() describes the problem. A failed launch returns
 *    LSA_ERR_HIP. Device-side values such as indices, counts and offsets are
 *    not range-checked beyond what each call states. A debug build of the
 *    library (LSA_DEBUG_CHECKS) checks every list entry that addresses a row
 *    against N_b; see lsa_debug_range_errors.
 *  - Sequences: B sequences are stored back to back. Sequence b owns rows
 *    [key_offsets[b], key_offsets[b+1]) of every per-entry buffer. Entry indices
 *    are sequence-local int32 values in [0, N_b), where
 *    N_b = key_offsets[b+1] - key_offsets[b].
 *  - Masks: bit (s % 64) of word mask_word_offsets[b] + s/64 is entry s of
 *    sequence b. Region b is exactly ceil(N_b/64) words, so no two sequences
 *    share a word. Bits at or beyond N_b are written as 0.
 *  - Layers: L indexer layers per call, 1 <= L <= LSA_MAX_LAYERS. The pages use
 *    three, at transformer layers 10, 12 and 20 ([BLOG] §4.2).
 */
#ifndef LSA_H
#define LSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LSA_MAX_LAYERS 8
#define LSA_MAX_HEADS 64
#define LSA_VERSION 2
#define LSA_GOLDEN_MAX_ROW (1 << 28)  /* entries per (token, layer) logit row */

typedef enum {
  LSA_F32 = 0,      /* IEEE binary32 */
  LSA_BF16 = 1,     /* bfloat16 */
  LSA_FP8_E4M3 = 2  /* OCP FP8 E4M3 ("e4m3fn"), keys only, one fp32 scale per entry */
} lsa_dtype;

typedef enum {
  LSA_OK = 0,
  LSA_ERR_INVALID_ARG = -1,
  LSA_ERR_UNSUPPORTED = -2,
  LSA_ERR_HIP = -3,
  LSA_ERR_WORKSPACE = -4
} lsa_status;

/* ------------------------------------------------------------------------
 * lsa_project: the indexer query and head gates of each layer ([BLOG] §3.1,
 * the down-projection, the up-projection and the head-routing weights).
 *
 *   c = h W^DQ (rank r), q = c W^IUQ viewed as [n_h, d_h] (head j is columns
 *   j*d_h ... (j+1)*d_h - 1), and w = h W^w.
 *
 * Weights are stored "out x in" (each output's weights are contiguous):
 *   w_dq  [r, d]         row n = column n of W^DQ
 *   w_iuq [n_h*d_h, r]   row m = column m of W^IUQ
 *   w_w   [n_h, d]       row j = column j of W^w
 * h is [B, d] row-major. h and all weights share `dtype` (LSA_F32 or LSA_BF16).
 * Outputs are fp32 and row-major: c_out [B, r], q_out [B, n_h, d_h],
 * w_out [B, n_h]. c_out is both an output and the input of the second stage,
 * so it must not alias the other buffers.
 * Supported shapes: 1 <= B <= 128; d and r multiples of 32 (of 4 for LSA_F32);
 * n_h * d_h a multiple of 16; 1 <= n_h <= LSA_MAX_HEADS. h, w_dq, w_iuq, w_w
 * and c_out must be 16-byte aligned.
 * Accumulation is fp32. With LSA_BF16, c enters the second product as
 * bf16 hi + lo, which keeps about 16 significant bits.
 * ---------------------------------------------------------------------- */
typedef struct {
  const void* h;      /* dev [B, d]          */
  const void* w_dq;   /* dev [r, d]          */
  const void* w_iuq;  /* dev [n_h*d_h, r]    */
  const void* w_w;    /* dev [n_h, d]        */
  float* c_out;       /* dev [B, r]   fp32   */
  float* q_out;       /* dev [B, n_h, d_h] fp32 */
  float* w_out;       /* dev [B, n_h] fp32   */
} lsa_proj_layer;

lsa_status lsa_project(const lsa_proj_layer* layers /* host [L] */, int32_t L, int32_t B,
                       int32_t d, int32_t r, int32_t n_h, int32_t d_h, lsa_dtype dtype,
                       hipStream_t stream);

/* ------------------------------------------------------------------------
 * lsa_pack_weights / lsa_project_packed: the same projection ([BLOG] §3.1)
 * with bf16 weights stored once in the layout the matrix cores read.
 *
 * The projection weights are constants of the model, so they can be
 * rearranged once (at load time) into a layout where every 1 KiB is one
 * wave's operand of one 16x16x32 MFMA step. A matrix of `rows` x K (out x in,
 * as for lsa_project) becomes ceil(rows/16) x (K/32) blocks of 1 KiB; block
 * (rb, ch) holds rows 16rb..16rb+15 and columns 32ch..32ch+31, and its
 * 16-byte unit l = 16*kg + m is row 16rb+m, columns 32ch+8kg .. 32ch+8kg+7.
 * Rows past the end are zero.
 *
 * lsa_pack_weights_size returns the bytes of the packed form of a rows x K
 * bf16 matrix (0 if K is not a positive multiple of 32 or rows < 1).
 * lsa_pack_weights writes it: w is dev [rows, K] bf16 (16-byte aligned),
 * out is dev memory of out_bytes >= lsa_pack_weights_size(rows, K). The
 * packed size must stay below 2^31 bytes. Pack W^DQ as (r, d), W^IUQ as
 * (n_h*d_h, r) and W^w as (n_h, d).
 *
 * lsa_project_packed takes lsa_proj_layer entries whose w_dq, w_iuq and w_w
 * point to packed matrices, and bf16 h. It computes the same c, q and w as
 * lsa_project (fp32 accumulation, c split into bf16 hi + lo for the second
 * product); the order of the fp32 sums differs, so results agree to rounding.
 * Supported: 1 <= B <= 32; d a multiple of 32; r a multiple of 64; n_h*d_h a
 * multiple of 64; 1 <= n_h <= LSA_MAX_HEADS. Errors as for lsa_project.
 * ---------------------------------------------------------------------- */
size_t lsa_pack_weights_size(int32_t rows, int32_t K);

lsa_status lsa_pack_weights(const void* w /* dev [rows, K] bf16 */, int32_t rows, int32_t K,
                            void* out /* dev */, size_t out_bytes, hipStream_t stream);

lsa_status lsa_project_packed(const lsa_proj_layer* layers /* host [L] */, int32_t L, int32_t B,
                              int32_t d, int32_t r, int32_t n_h, int32_t d_h, hipStream_t stream);

/* ------------------------------------------------------------------------
 * lsa_score_select: the lookahead index score and the loading rule
 * ([BLOG] §3.1; [HYPER] 方法: entries whose score reaches or exceeds the
 * threshold are fetched).
 *
 *   x_s = sum_j w_j * ReLU(q_j . K_s),   I_s = 1 / (1 + exp(-x_s)),
 *   selected  <=>  I_s >= threshold  <=>  x_s >= ln(threshold / (1 - threshold)).
 *
 * The comparison is made on the fp32 logit against the logit threshold, which
 * is computed in double precision on the host (exactly 0 for threshold 0.5),
 * so rounding in the sigmoid never decides membership. A sum that is exactly
 * zero (every head's dot product <= 0, or every gate 0) selects the entry.
 * Keys: [rows, d_h], in LSA_F32, LSA_BF16 or LSA_FP8_E4M3. For FP8 the key is
 * key_scale[s] * e4m3(K8_s), and the scale must be positive and finite. One key
 * serves all heads. q and w come from lsa_project or any other source: q is
 * [B, n_h, d_h] fp32 and w is [B, n_h] fp32. score_out, if non-NULL, receives I_s
 * as fp32 for every entry. mask_out receives the selection bits (see "Masks").
 * Supported: d_h in {32, 64, 128}; 1 <= n_h <= 64; 0 < threshold < 1.
 * Sequences with N_b = 0 are allowed and write nothing.
 * Precision: with fp32 keys the contraction is fp32. With bf16 or fp8 keys, q
 * enters the bf16 matrix cores as hi + lo parts (about 16 significant bits),
 * with fp32 accumulation.
 * ---------------------------------------------------------------------- */
typedef struct {
  const float* q;          /* dev [B, n_h, d_h] fp32 */
  const float* w;          /* dev [B, n_h] fp32 */
  const void* keys;        /* dev [rows, d_h] */
  const float* key_scale;  /* dev [rows] fp32 for LSA_FP8_E4M3, else NULL */
  uint64_t* mask_out;      /* dev, words [mask_word_offsets[0], mask_word_offsets[B]) */
  float* score_out;        /* dev [rows] fp32, or NULL */
} lsa_score_layer;

lsa_status lsa_score_select(const lsa_score_layer* layers /* host [L] */, int32_t L, int32_t B,
                            const int64_t* key_offsets /* dev [B+1] */,
                            const int64_t* key_offsets_host /* host [B+1] */,
                            const int64_t* mask_word_offsets /* dev [B+1] */,
                            const int64_t* mask_word_offsets_host /* host [B+1] */,
                            int32_t n_h, int32_t d_h, lsa_dtype key_dtype, float threshold,
                            hipStream_t stream);

/* lsa_score_select_ex: lsa_score_select with an explicit choice of launch
 * variant, for tests and tuning. lsa_score_select is this call with
 * options == NULL, which means every field 0. Results agree with
 * lsa_score_select's to the precision stated there; masks outside rounding of
 * the threshold are identical.
 *   kernel       LSA_SCORE_KERNEL_AUTO (0): one wave per 32-entry tile for bf16
 *                and fp8 keys, the wave-pair kernel for fp32 keys;
 *                LSA_SCORE_KERNEL_STREAM (1): one wave per tile (bf16 keys with
 *                d_h 32/64/128, fp8 keys with d_h 64/128; else
 *                LSA_ERR_UNSUPPORTED); LSA_SCORE_KERNEL_PAIRS (2): two waves
 *                share each tile (every key dtype).
 *   chunk_words  mask words (64 entries each) a wave takes at a time in the
 *                one-wave-per-tile kernel: 0 (default, 2) or 2..64.
 *   ring         LDS ring depth of that kernel in half tiles: 0 (default), 4,
 *                or 8 (8 only for rows of at most 128 bytes).
 *   guard        1 (one-wave-per-tile kernel, masks only): score each 32-entry
 *                tile with the bf16 hi part of q alone first, and complete
 *                with the lo part only the tiles in which some entry's logit
 *                lies within a computed bound of the threshold (the bound
 *                covers everything the lo part can change), so every decision
 *                equals the full computation's. Ignored when a layer asks for
 *                scores. 0 (default): every tile with hi + lo.
 * Other values return LSA_ERR_INVALID_ARG. */
enum { LSA_SCORE_KERNEL_AUTO = 0, LSA_SCORE_KERNEL_STREAM = 1, LSA_SCORE_KERNEL_PAIRS = 2 };
typedef struct {
  int32_t kernel;
  int32_t chunk_words;
  int32_t ring;
  int32_t guard;
} lsa_score_options;

lsa_status lsa_score_select_ex(const lsa_score_layer* layers /* host [L] */, int32_t L, int32_t B,
                               const int64_t* key_offsets /* dev [B+1] */,
                               const int64_t* key_offsets_host /* host [B+1] */,
                               const int64_t* mask_word_offsets /* dev [B+1] */,
                               const int64_t* mask_word_offsets_host /* host [B+1] */,
                               int32_t n_h, int32_t d_h, lsa_dtype key_dtype, float threshold,
                               const lsa_score_options* options /* host, or NULL */, hipStream_t stream);

/* ------------------------------------------------------------------------
 * lsa_union_compact: OR-mode routing over the indexer layers. Entry s is
 * fetched if any layer selected it ([BLOG] §4.2; [HYPER] 方法). The union is
 * then compacted into the subset C^MemComp as an ascending list of
 * sequence-local indices.
 *
 * idx_out region b starts at key_offsets[b] and holds up to N_b int32 values.
 * The first count_out[b] are written in ascending order and the rest are left
 * untouched. union_mask_out (optional) receives the OR of the masks in the
 * mask layout.
 * ---------------------------------------------------------------------- */
lsa_status lsa_union_compact(const uint64_t* const* masks /* host [L] of dev pointers */, int32_t L,
                             int32_t B, const int64_t* key_offsets /* dev [B+1] */,
                             const int64_t* key_offsets_host /* host [B+1] */,
                             const int64_t* mask_word_offsets /* dev [B+1] */,
                             const int64_t* mask_word_offsets_host /* host [B+1] */,
                             int32_t* idx_out /* dev [rows] */, int32_t* count_out /* dev [B] */,
                             uint64_t* union_mask_out /* dev or NULL */, hipStream_t stream);

/* ------------------------------------------------------------------------
 * lsa_topk: the native Lightning Indexer's fine selection inside the loaded
 * subset ([BLOG] §3.2 second level; §2.2 for the native score, which is a
 * head-gated ReLU sum with no sigmoid).
 *
 * For each layer l and sequence b, and for each s in the subset
 * idx[key_offsets[b] .. key_offsets[b] + count[b]), the call scores
 *   y_s = sum_j w'_j * ReLU(q'_j . K^l_s),
 * with the layer's native query q' [B, n_h, d_h] and gates w' [B, n_h]. It
 * keeps the min(k, count[b]) entries that come first in the order (-y_s, s),
 * so ties go to the lower index. topk_idx_out[b*k .. b*k + k) receives them in
 * ascending index order, padded with -1. topk_score_out (optional) receives
 * the matching y values, padded with -inf. topk_count_out[l*B + b] receives
 * min(k, count[b]). idx must be ascending within each sequence, which is what
 * lsa_union_compact writes.
 *
 * The workspace must hold at least lsa_topk_workspace_size(...) bytes of
 * device memory, 256-byte aligned. Its contents on entry do not matter. It
 * holds the subset scores, one fp32 per (layer, row), and per (layer,
 * sequence) a 2048-bin count of the scores by their top 11 bits (sign,
 * exponent and two mantissa bits of an order-preserving key), which the
 * selection uses to find the k-th score's bin without sampling. The counts
 * are kept only when some sequence has more than 131,072 rows; otherwise the
 * selection counts the bins of each list itself and that part of the
 * workspace is left untouched. Supported:
 * 1 <= k <= 65536; B <= 4096; the key dtypes and head shapes of
 * lsa_score_select.
 * ---------------------------------------------------------------------- */
typedef struct {
  const float* q;          /* dev [B, n_h, d_h] fp32 (native query q') */
  const float* w;          /* dev [B, n_h] fp32 (native gates w') */
  const void* keys;        /* dev [rows, d_h] (this layer's K^l) */
  const float* key_scale;  /* dev [rows] for LSA_FP8_E4M3, else NULL */
  int32_t* topk_idx_out;   /* dev [B, k] */
  float* topk_score_out;   /* dev [B, k] or NULL */
} lsa_topk_layer;

size_t lsa_topk_workspace_size(int32_t L, int32_t B, int64_t total_rows, int32_t k);

lsa_status lsa_topk(const lsa_topk_layer* layers /* host [L] */, int32_t L, int32_t B,
                    const int64_t* key_offsets /* dev [B+1] */,
                    const int64_t* key_offsets_host /* host [B+1] */,
                    const int32_t* idx /* dev [rows] */, const int32_t* count /* dev [B] */,
                    int32_t n_h, int32_t d_h, lsa_dtype key_dtype, int32_t k,
                    int32_t* topk_count_out /* dev [L, B] */, void* workspace /* dev */,
                    size_t workspace_bytes, hipStream_t stream);

/* The two stages of lsa_topk as separate calls, so that other work can be
 * ordered between them (the scoring streams the subset's keys from HBM; the
 * selection runs one workgroup per (layer, sequence) and is latency-bound).
 * lsa_topk_score writes the subset scores into the workspace and reads only
 * q, w, keys and key_scale of each layer. lsa_topk_select reads them back and
 * writes topk_idx_out, topk_score_out and topk_count_out. Run them in that
 * order with the same lists, counts and workspace (on one stream, or with the
 * selection ordered after the scoring). lsa_topk is the two in sequence. */
lsa_status lsa_topk_score(const lsa_topk_layer* layers /* host [L] */, int32_t L, int32_t B,
                          const int64_t* key_offsets /* dev [B+1] */,
                          const int64_t* key_offsets_host /* host [B+1] */,
                          const int32_t* idx /* dev [rows] */, const int32_t* count /* dev [B] */,
                          int32_t n_h, int32_t d_h, lsa_dtype key_dtype, void* workspace /* dev */,
                          size_t workspace_bytes, hipStream_t stream);

lsa_status lsa_topk_select(const lsa_topk_layer* layers /* host [L] */, int32_t L, int32_t B,
                           const int64_t* key_offsets /* dev [B+1] */,
                           const int64_t* key_offsets_host /* host [B+1] */,
                           const int32_t* idx /* dev [rows] */, const int32_t* count /* dev [B] */,
                           int32_t k, int32_t* topk_count_out /* dev [L, B] */, void* workspace /* dev */,
                           size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * lsa_topk_step: the native indexer's top-k at one decode step, over the
 * subset that is already resident ([BLOG] §3.2: the memory indexer loads
 * C^MemComp once per trigger, and inside it the native Lightning Indexer
 * selects its top-k at every decode step; [HYPER] 方法).
 *
 * Same result and arguments as lsa_topk, except that each layer's `keys`
 * points to that layer's subset keys packed in list order: row
 * P_b + i is the key of list entry i of sequence b, where
 * P_b = count[0] + ... + count[b-1] (lsa_gather in packed mode, with the
 * layer's key array as the pool, row_bytes = d_h times the key size, and the
 * union lists, writes exactly this). The packed rows are read contiguously,
 * with no index load before them. For fp8 keys, key_scale is still the full
 * per-entry scale array of the layer ([rows], read through the lists). q and
 * w are the step's native query and gates. Call it once per decode step; the
 * lists, counts and packed keys stay the same over the steps of a trigger.
 * Supported: as lsa_topk, with B <= 1024 and at most 2^31 - 1 list entries
 * over all sequences. The workspace is lsa_topk_workspace_size(L, B, rows, k).
 * ---------------------------------------------------------------------- */
lsa_status lsa_topk_step(const lsa_topk_layer* layers /* host [L]; keys = packed subset keys */, int32_t L,
                         int32_t B, const int64_t* key_offsets /* dev [B+1] */,
                         const int64_t* key_offsets_host /* host [B+1] */,
                         const int32_t* idx /* dev [rows] */, const int32_t* count /* dev [B] */,
                         int32_t n_h, int32_t d_h, lsa_dtype key_dtype, int32_t k,
                         int32_t* topk_count_out /* dev [L, B] */, void* workspace /* dev */,
                         size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * lsa_topk_step_noalloc: lsa_topk_step for callers that cannot allocate or
 * hold device memory of their own: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation. It takes no workspace and allocates
 * nothing; its scratch (the subset scores and the score histograms) is a fixed
 * array of LSA_NOALLOC_SCRATCH_BYTES in device memory, one copy on every GPU
 * the library runs on, held until the process ends.
 *
 * Arguments, results and errors are those of lsa_topk_step. A call whose
 * scratch, lsa_topk_workspace_size(L, B, key_offsets_host[B], k), exceeds
 * LSA_NOALLOC_SCRATCH_BYTES returns LSA_ERR_UNSUPPORTED before any HIP call.
 * Each call clears what it needs cleared, and leaves the array holding its own
 * scratch. Calls on one GPU share the array: two calls that may overlap in
 * time on one GPU (on different streams, or from different threads without
 * ordering) race and give wrong results; order them on one stream.
 * ---------------------------------------------------------------------- */
#define LSA_NOALLOC_SCRATCH_BYTES (32 << 20)
lsa_status lsa_topk_step_noalloc(const lsa_topk_layer* layers /* host [L]; keys = packed subset keys */,
                                 int32_t L, int32_t B, const int64_t* key_offsets /* dev [B+1] */,
                                 const int64_t* key_offsets_host /* host [B+1] */,
                                 const int32_t* idx /* dev [rows] */, const int32_t* count /* dev [B] */,
                                 int32_t n_h, int32_t d_h, lsa_dtype key_dtype, int32_t k,
                                 int32_t* topk_count_out /* dev [L, B] */, hipStream_t stream);

/* ------------------------------------------------------------------------
 * lsa_gather: load the selected entries' compressed-KV rows into a compact
 * device buffer ([HYPER] 方法: the subset C^MemComp is loaded into GPU memory).
 * Here the pool is already in device memory, so this is an HBM-to-HBM row copy.
 *
 * Row i < count[b] of sequence b is pool row pool_row_offsets[b] + idx[idx_offsets[b] + i].
 * It is copied byte for byte, as row_bytes bytes, to output row o_b + i:
 *   - packed mode (out_row_offsets == NULL): o_b = count[0] + ... + count[b-1].
 *     The sequences are packed back to back, which is the compact buffer.
 *   - explicit mode: o_b = out_row_offsets[b], and at most
 *     out_row_offsets[b+1] - out_row_offsets[b] rows are written for b.
 * Output rows at or beyond out_capacity_rows are never written. Rows that do
 * not fit are dropped. row_bytes must be a positive multiple of 16. pool and
 * out must be 16-byte aligned. idx values must lie in [0, N_b) of the pool
 * region; this is not checked on the device.
 * ---------------------------------------------------------------------- */
lsa_status lsa_gather(const void* pool /* dev */, int64_t row_bytes, int32_t B,
                      const int64_t* pool_row_offsets /* dev [B+1] */,
                      const int64_t* pool_row_offsets_host /* host [B+1] */,
                      const int32_t* idx /* dev */, const int64_t* idx_offsets /* dev [B] */,
                      const int32_t* count /* dev [B] */, void* out /* dev */,
                      const int64_t* out_row_offsets /* dev [B+1] or NULL */,
                      int64_t out_capacity_rows, hipStream_t stream);

/* ------------------------------------------------------------------------
 * lsa_fetch_host: the same row copy as lsa_gather, from a cold pool kept in
 * host memory ([HYPER] 方法 and [BLOG] §3: the subset C^MemComp is loaded from
 * the CPU-side pool into GPU memory). The device reads the selected rows
 * straight from pinned host memory over the host link, with no staging copy,
 * and writes them into `out` in device memory.
 *
 * Arguments and layout are those of lsa_gather, except:
 *   - pool_host must point into pinned host memory the device can read
 *     (allocated with hipHostMalloc or hipHostAlloc); pageable memory returns
 *     LSA_ERR_INVALID_ARG. The caller keeps it alive until the stream has
 *     passed the call.
 * The copy is bit-exact. Its speed is that of the host link, not of HBM.
 * ---------------------------------------------------------------------- */
lsa_status lsa_fetch_host(const void* pool_host /* pinned host */, int64_t row_bytes, int32_t B,
                          const int64_t* pool_row_offsets /* dev [B+1] */,
                          const int64_t* pool_row_offsets_host /* host [B+1] */,
                          const int32_t* idx /* dev */, const int64_t* idx_offsets /* dev [B] */,
                          const int32_t* count /* dev [B] */, void* out /* dev */,
                          const int64_t* out_row_offsets /* dev [B+1] or NULL */,
                          int64_t out_capacity_rows, hipStream_t stream);

/* ------------------------------------------------------------------------
 * lsa_golden_labels: golden-label mining, the training targets of the memory
 * indexer ([HYPER] 数据集 (Dataset); [BLOG] §4.1 "Golden Label 怎么造"; the
 * gist.science summary, §2.2). For each token i of a lookahead window of T
 * tokens and each of L layers, the raw indexer logits y[i][l][s] over the
 * token's n_valid[i] preceding compressed entries are turned into a softmax,
 * and the top-p nucleus of that distribution is kept. An entry is golden for
 * token i when at least `theta` layers keep it; the window's label set is the
 * union of the tokens' golden sets. The pages use L = 21, p = 0.6, theta = 3.
 *
 * Nucleus: entries in descending logit order, equal logits by ascending entry
 * index; an entry is kept while the mass of the entries before it is below
 * top_p (so the entry that reaches top_p is kept, and the top entry always is).
 *
 *   logits          dev fp32 [T][L][row_stride]; row (i, l) holds token i's
 *                   logits in its first n_valid[i] entries (finite values);
 *                   the rest of the row is never read.
 *   n_valid         dev int32 [T]; values are clamped to [0, row_stride].
 *   top_p           in (0, 1].  theta >= 1 (theta > L gives an empty set).
 *   row_mask_out    dev u64 [T * L][W], W = ceil(row_stride / 64): the nucleus
 *                   of row (i, l) as bits (bit s % 64 of word s / 64); bits at
 *                   or beyond n_valid[i] are 0.
 *   nucleus_size_out  dev int32 [T * L] or NULL: kept entries per row.
 *   token_golden_out  dev u64 [T][W] or NULL: token i's golden entries.
 *   golden_out      dev u64 [W]: the window's label set.
 *   workspace       dev scratch of lsa_golden_workspace_size(T, L, row_stride)
 *                   bytes, 16-byte aligned; its contents need no clearing and
 *                   are not meaningful to the caller. Calls that share one
 *                   workspace must be ordered on a stream.
 * Probabilities are accumulated in fp64 from fp32 exponentials relative to the
 * row maximum; an entry whose preceding mass is within about 1e-5 of top_p
 * may fall either way. Requires 1 <= L <= 64, 1 <= row_stride <=
 * LSA_GOLDEN_MAX_ROW; logits 4-byte and the mask buffers 8-byte aligned.
 * A missing or short workspace returns LSA_ERR_WORKSPACE.
 * ---------------------------------------------------------------------- */
size_t lsa_golden_workspace_size(int32_t T, int32_t L, int64_t row_stride);
lsa_status lsa_golden_labels(const float* logits /* dev */, int64_t row_stride, int32_t T, int32_t L,
                             const int32_t* n_valid /* dev [T] */, float top_p, int32_t theta,
                             uint64_t* row_mask_out /* dev [T*L][W] */,
                             int32_t* nucleus_size_out /* dev [T*L] or NULL */,
                             uint64_t* token_golden_out /* dev [T][W] or NULL */,
                             uint64_t* golden_out /* dev [W] */, void* workspace /* dev */,
                             size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * lsa_train_step: one training step of a memory-indexer layer ([BLOG] §4
 * "训练" (training); [HYPER] 方法 (Method); the gist.science summary names the
 * same loss). The compressed index keys are frozen; the query side's
 * projections are trained with a focal binary cross-entropy on the selection
 * score against the golden labels.
 *
 *   c = h W^DQ, q = c W^IUQ viewed as [n_h, d_h], w = h W^w   (as lsa_project)
 *   x_s = sum_j w_j ReLU(q_j . K_s),  p_s = sigmoid(x_s)       ([BLOG] §3.1)
 *   loss = mean over every entry s of every sequence of
 *          -alpha (1 - p_s)^gamma log p_s          if s is golden,
 *          -(1 - alpha) p_s^gamma log(1 - p_s)     otherwise.
 * Outputs are the loss and its gradients with respect to the three weight
 * matrices, in the weights' own "out x in" layouts.
 *
 *   h, w_dq, w_iuq, w_w  dev bf16, the lsa_project layouts ([B, d], [r, d],
 *                   [n_h*d_h, r], [n_h, d]); 16-byte aligned.
 *   keys            dev bf16 [rows][d_h], the selection path's layout.
 *   key_offsets, mask_word_offsets (dev and host copies): as lsa_score_select.
 *   labels          dev u64 bit masks (8-byte aligned) in the lsa_score_select mask layout: bit
 *                   s % 64 of word mask_word_offsets[b] + s / 64 is 1 when entry s
 *                   of sequence b is golden. Bits past N_b are ignored.
 *   gamma >= 0, alpha in [0, 1]  the focal constants (2 and 0.25 usually).
 *   loss_out        dev fp32 [1].
 *   g_dq            dev fp32 [r, d];  g_iuq  dev fp32 [n_h*d_h, r];
 *   g_w             dev fp32 [n_h, d]. Every element is written. The gradients
 *                   must be 16-byte aligned.
 *   workspace       dev scratch of lsa_train_workspace_size(B,
 *                   key_offsets_host, r) bytes, 16-byte aligned; it needs no
 *                   clearing. Calls that share one workspace must be ordered.
 * Precision: the projections as lsa_project with LSA_BF16; in the key scan q
 * and the per-(entry, head) gradient coefficients enter bf16 MFMAs as hi + lo
 * pairs (about 16 significant bits), with fp32 accumulation. The loss is summed
 * in fp64 per scan block (a run of at least 256 entries of one sequence). A
 * score within rounding of 0 may fall on
 * either side of the ReLU kink.
 * Supported: n_h = 64, d_h = 128, 1 <= B <= 32, d and r positive multiples of
 * 32, N_b < 2^23 entries per sequence. A sequence with no entries adds nothing;
 * with no entries at all the loss and the gradients are 0.
 * A missing or short workspace returns LSA_ERR_WORKSPACE.
 * ---------------------------------------------------------------------- */
size_t lsa_train_workspace_size(int32_t B, const int64_t* key_offsets_host /* host [B+1] */, int32_t r);
lsa_status lsa_train_step(const void* h /* dev */, const void* w_dq /* dev */, const void* w_iuq /* dev */,
                          const void* w_w /* dev */, const void* keys /* dev */,
                          const int64_t* key_offsets /* dev [B+1] */,
                          const int64_t* key_offsets_host /* host [B+1] */, const uint64_t* labels /* dev */,
                          const int64_t* mask_word_offsets /* dev [B+1] */,
                          const int64_t* mask_word_offsets_host /* host [B+1] */, int32_t B, int32_t d, int32_t r,
                          int32_t n_h, int32_t d_h, float gamma, float alpha, float* loss_out /* dev [1] */,
                          float* g_dq /* dev [r, d] */, float* g_iuq /* dev [n_h*d_h, r] */,
                          float* g_w /* dev [n_h, d] */, void* workspace /* dev */, size_t workspace_bytes,
                          hipStream_t stream);

/* ------------------------------------------------------------------------
 * lsa_debug_range_errors: in a debug build (compiled with LSA_DEBUG_CHECKS=1),
 * the number of out-of-range list entries that the gather, the cold-pool
 * fetch and the top-k scoring of gathered rows have met since the previous
 * call. Such an entry (an index outside [0, N_b) of its sequence) is counted
 * and its row is not read: its gathered row is not written, and its top-k score
 * is that of an all-zero key. One entry may be counted more than once. The
 * count is cleared by the call.
 *
 * Unlike every other call it synchronises: it waits for `stream` and copies the
 * count to the host. Counts are per device and shared by all streams.
 * A release build returns LSA_ERR_UNSUPPORTED and leaves *count_out alone.
 * ---------------------------------------------------------------------- */
lsa_status lsa_debug_range_errors(hipStream_t stream, int64_t* count_out /* host [1] */);

/* Text describing the last non-OK status returned on the calling thread. */
const char* lsa_last_error(void);

/* LSA_VERSION of the built library. */
int32_t lsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LSA_H */
