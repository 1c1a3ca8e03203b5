/*
 * fmha_mqa.h — multi-query attention forward for AMD MI355X (gfx950).
 *
 * C ABI of libfmha_mqa.so.  Every pointer argument named q/k/v/kv_idx/out/lse/
 * o_parts/lse_parts/workspace is a DEVICE pointer allocated and owned by the
 * caller; the library never allocates, frees or synchronises, keeps no state
 * between calls, and launches all work asynchronously on the given stream
 * (a hipStream_t passed as void*; NULL = the default stream).  Tensors are
 * row-major and contiguous.  No C++ exception crosses this boundary: every
 * function returns an fmha_status code.  Validation happens before any launch:
 * a validation error (FMHA_ERR_INVALID_ARG, _UNSUPPORTED, _ALIGNMENT,
 * _WORKSPACE) means nothing was enqueued.  FMHA_ERR_LAUNCH means the HIP
 * runtime refused a launch; when a call makes several launches, the ones
 * before it may already be on the stream (they write only the caller's
 * workspace or outputs).  Device faults, as for any HIP work, surface at the
 * caller's next synchronisation.
 *
 * The operation is the fused attention forward of a DeepSeek-V4-style decoder
 * as described on the dev-log pages of the "nvfp4-megamoe-kernel" project:
 *   - QK^T -> softmax -> PV -> output, with the 1/sqrt(hd) scale applied in the
 *     softmax to the unscaled dot product: page "CURRENT ISSUE: UMMA FMHA — Full
 *     Pipeline + Production", sections "What's working" and "Key lessons from
 *     this session";
 *   - multi-query layout, K/V shared by every query head: page "May 24, 2026 —
 *     Session Start Plan", section 3 "Start D2: Multi-Query Grid";
 *   - O together with the row log-sum-exp: same page, "D1 Status Summary";
 *   - more than one KV tile needs the running O rescaled: same page, section 2
 *     "Test O Rescale at s_k > 128" and "Key Numbers" (8 tiles at top_k 1024);
 *   - parts merged by O = sum_i exp(lse_i) O_i / sum_i exp(lse_i): page
 *     "CURRENT ISSUE: UMMA FMHA — Full Pipeline + Production", "Next steps" 4;
 *   - s_k = top_k keys selected from a KV store: "Key Numbers" and the
 *     dsv4/kernels/cuda commit log (KV row gather, 32768-row compressed pool).
 *
 * Definition (per output row r = (b, t, h), natural log):
 *   x_j   = scale * sum_d q[b,t,h,d] * K_j[d]
 *   out[r] = sum_j softmax(x)_j * V_j          (normalised over the row's keys)
 *   lse[r] = ln sum_j exp(x_j)
 * with K_j, V_j = k[b,j], v[b,j] (dense) or k[kv_idx[b,t,j]], v[kv_idx[b,t,j]]
 * (gather).  A row with no keys has out = 0 and lse = -inf.
 */
#ifndef FMHA_MQA_H
#define FMHA_MQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FMHA_OK = 0,
  FMHA_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad dtype/scale/splits */
  FMHA_ERR_UNSUPPORTED = 2, /* head dim not in {64, 128, 256, 512}; more than 2^31-1 rows;
                               K/V (s_k rows dense, pool_rows gather) over 2 GiB */
  FMHA_ERR_ALIGNMENT = 3,   /* a tensor pointer not 16-byte aligned (lse: 4-byte) */
  FMHA_ERR_WORKSPACE = 4,   /* workspace missing, too small or misaligned */
  FMHA_ERR_LAUNCH = 5,      /* the HIP runtime rejected a kernel launch */
  FMHA_ERR_SCRATCH_LIMIT = 6 /* fmha_mqa_fwd_noalloc: the split partials need more than
                               FMHA_SCRATCH_BYTES */
} fmha_status;

/* Size of the library's static per-GPU scratch buffer (fmha_mqa_fwd_noalloc). */
#define FMHA_SCRATCH_BYTES (64u << 20)

typedef enum { FMHA_F32 = 0, FMHA_BF16 = 1 } fmha_dtype;

/* Bytes of workspace fmha_mqa_fwd needs for num_splits > 1 (0 when
 * num_splits == 1): partial outputs [num_splits, B*T*n_h, hd] sized for fp32
 * (they are stored as bf16 when the output is bf16, in the same region) and
 * fp32 partial LSEs [num_splits, B*T*n_h], each region 256-byte aligned.
 * Returns 0 as well for invalid arguments. */
size_t fmha_mqa_workspace_bytes(int B, int T, int n_h, int hd, int num_splits);

/* Attention forward.
 *  q        bf16 [B, T, n_h, hd]
 *  k, v     bf16 [B, s_k, hd] when kv_idx == NULL (dense: every query head of
 *           batch b reads the same K/V rows), else bf16 pools [pool_rows, hd]
 *  kv_idx   NULL, or int32 [B, T, s_k]: token (b, t) attends to pool rows
 *           kv_idx[b, t, 0..s_k-1].  An entry outside [0, pool_rows) is never
 *           read; that key is masked out (weight 0).
 *  out      [B, T, n_h, hd] of out_dtype (FMHA_F32 or FMHA_BF16, RNE rounding)
 *  lse      fp32 [B, T, n_h], natural log
 *  B, T, n_h >= 0 (a zero gives an immediate FMHA_OK); s_k >= 0 (0: every row
 *           empty, k/v/kv_idx may be NULL); hd in {64, 128, 256, 512};
 *  pool_rows  rows of the k/v pools (gather only; ignored when kv_idx == NULL)
 *  scale    finite and > 0 (e.g. 1/sqrt(hd))
 *  num_splits  1: one pass over the keys.  > 1 (at most max(s_k, 1)): split-KV —
 *           the keys are cut into contiguous chunks of ceil(s_k/num_splits);
 *           each chunk's normalised partial O and LSE go to the workspace and a
 *           second kernel merges them (see fmha_lse_merge) into out/lse.
 *  workspace   device memory of >= fmha_mqa_workspace_bytes(...) bytes,
 *           16-byte aligned; may be NULL when num_splits == 1.
 * q, k, v, out, workspace must be 16-byte aligned; kv_idx and lse 4-byte. */
int fmha_mqa_fwd(const void* q, const void* k, const void* v,
                 const int32_t* kv_idx, void* out, float* lse,
                 int B, int T, int n_h, int s_k, int hd, int pool_rows,
                 float scale, int out_dtype, int num_splits,
                 void* workspace, size_t workspace_bytes, void* stream);

/* fmha_mqa_fwd for callers that cannot allocate device memory — code under HIP
 * graph capture, serving loops and harnesses that forbid hipMalloc: the same
 * forward without the workspace arguments.  A split-KV call (num_splits > 1)
 * keeps its partials in a static buffer of FMHA_SCRATCH_BYTES that the library
 * holds on each GPU it runs on until the process ends; the call itself
 * allocates nothing.  Arguments, layouts and results as fmha_mqa_fwd.
 *  Limit: the partials (fmha_mqa_workspace_bytes(B, T, n_h, hd, num_splits)
 *  bytes) must fit in FMHA_SCRATCH_BYTES, else FMHA_ERR_SCRATCH_LIMIT and
 *  nothing is enqueued (e.g. B*T*n_h = 4096 rows at hd 256 allow 15 splits).
 *  Every call on one GPU shares that GPU's buffer: calls that may overlap on
 *  one GPU (different streams, or several host threads) race and must be
 *  serialised by the caller; calls on one stream are ordered by it.
 *  FMHA_ERR_LAUNCH is also returned if the buffer's device address cannot be
 *  obtained (looked up once per GPU, on the first split-KV call there). */
int fmha_mqa_fwd_noalloc(const void* q, const void* k, const void* v,
                         const int32_t* kv_idx, void* out, float* lse,
                         int B, int T, int n_h, int s_k, int hd, int pool_rows,
                         float scale, int out_dtype, int num_splits, void* stream);

/* fmha_mqa_fwd with an attention sink joined to every row (page "May 24, 2026 —
 * Session Start Plan" names a "sink merge" — File Map, D1 Status Summary D5b —
 * without printing it; the reading taken: one extra logit per query head whose
 * value vector is zero).  For row (b, t, h) with lse over its keys:
 *   lse' = ln(exp(lse) + exp(sink[h])),  out' = out * exp(lse - lse').
 *  sink   fp32 [n_h], natural-log units like lse; -inf = no sink for that head;
 *         must not be NULL.  4-byte aligned.
 * Everything else as fmha_mqa_fwd.  The sink is applied once per row, in the
 * epilogue (num_splits == 1) or in the merge (split-KV), before the output is
 * rounded to out_dtype.  A row without keys gets out = 0, lse = sink[h]. */
int fmha_mqa_fwd_sink(const void* q, const void* k, const void* v,
                      const int32_t* kv_idx, void* out, float* lse,
                      int B, int T, int n_h, int s_k, int hd, int pool_rows,
                      float scale, int out_dtype, int num_splits,
                      void* workspace, size_t workspace_bytes, void* stream,
                      const float* sink);

/* The split-KV forward without its merge: the normalised partial O and the
 * LSE of every split, in fp32, written to caller memory (the split-KV + merge
 * plan of page "CURRENT ISSUE: UMMA FMHA — Full Pipeline + Production", "Next
 * steps" item 4, with the merge left to the caller).  Several calls may write
 * disjoint planes of one [n_parts, rows, hd] buffer, e.g. one call per key
 * source, so that a single fmha_lse_merge combines all of them.
 *  o_parts    fp32 [num_splits, B*T*n_h, hd]: plane i = attention over split
 *             i's keys, normalised over them (O = 0 for a split without keys)
 *  lse_parts  fp32 [num_splits, B*T*n_h], natural log (-inf: split without keys)
 * Everything else as fmha_mqa_fwd (num_splits may be 1: one plane).
 * o_parts 16-byte aligned, lse_parts 4-byte. */
int fmha_mqa_fwd_partials(const void* q, const void* k, const void* v,
                          const int32_t* kv_idx, float* o_parts, float* lse_parts,
                          int B, int T, int n_h, int s_k, int hd, int pool_rows,
                          float scale, int num_splits, void* stream);

/* One key source of fmha_mqa_fwd_sources_partials: the arguments that
 * fmha_mqa_fwd_partials takes per call.
 *  k, v        bf16: dense [B, s_k, hd] (kv_idx NULL), or pools [pool_rows, hd]
 *  kv_idx      NULL, or int32 [B, T, s_k] pool rows (entries outside
 *              [0, pool_rows) are masked, as in fmha_mqa_fwd)
 *  s_k         keys per query row from this source (>= 0)
 *  pool_rows   gather: rows in the pools (>= 1); dense: ignored
 *  num_splits  1 .. max(s_k, 1): this source's partial planes */
typedef struct fmha_kv_source {
  const void* k;
  const void* v;
  const int32_t* kv_idx;
  int s_k;
  int pool_rows;
  int num_splits;
} fmha_kv_source;

/* The partials of several key sources in one call: the split planes of
 * sources[0], then those of sources[1], ..., in one buffer, so that one
 * fmha_lse_merge over all of them gives attention over the union of the
 * sources' keys (page "May 24, 2026 — Session Start Plan": the top-k rows
 * gathered from the compressed pool, File Map and Key Numbers; a sliding
 * window of recent keys beside them is the second source this serves).
 *  sources    n_sources >= 1 entries, read during the call only
 *  o_parts    fp32 [sum of num_splits, B*T*n_h, hd], 16-byte aligned
 *  lse_parts  fp32 [sum of num_splits, B*T*n_h], 4-byte aligned
 * Every plane is what fmha_mqa_fwd_partials writes for that source and split
 * (bit for bit).  At hd 512, with at most 4 sources whose splits have at most
 * 1024 keys each, all sources' splits run in one kernel launch; otherwise one
 * launch per source.  Every source is validated before anything is enqueued;
 * errors as fmha_mqa_fwd_partials (FMHA_ERR_INVALID_ARG also for n_sources < 1
 * or sources NULL). */
int fmha_mqa_fwd_sources_partials(const void* q, const fmha_kv_source* sources,
                                  int n_sources, float* o_parts, float* lse_parts,
                                  int B, int T, int n_h, int hd, float scale,
                                  void* stream);

/* The same sink applied in place to finished rows (for results already merged
 * from several sources): for r in [0, rows), with h = r % n_h,
 *   lse[r] <- ln(exp(lse[r]) + exp(sink[h])),  out[r, :] *= exp(lse_old - lse_new).
 *  out   [rows, hd] of out_dtype (bf16 rows are rounded again after scaling)
 *  lse   fp32 [rows], natural log;  sink fp32 [n_h]
 * rows >= 0, n_h >= 1, hd >= 4 and a multiple of 4; out 16-byte aligned
 * (8-byte for bf16), lse and sink 4-byte. */
int fmha_attention_sink(void* out, float* lse, const float* sink, int rows,
                        int n_h, int hd, int out_dtype, void* stream);

/* Measurement helper, not part of the attention: the gather-only floor of the
 * top-k row gather (the data movement the gathered attention cannot avoid:
 * token (b, t) reads pool rows kv_idx[b, t, 0..s_k-1] of k and of v, every
 * 16-byte chunk once, with no arithmetic on them).  Writes the XOR of all words
 * a token read to out[b*T + t] (so no load can be dropped; an entry outside
 * [0, pool_rows) reads nothing).
 *  k, v   bf16 pools [pool_rows, hd], hd in {64, 128, 256, 512}, 16-byte aligned
 *  kv_idx int32 [B, T, s_k];  out uint32 [B*T], 4-byte aligned. */
int fmha_gather_floor(const void* k, const void* v, const int32_t* kv_idx, uint32_t* out,
                      int B, int T, int s_k, int hd, int pool_rows, void* stream);

/* Measurement helper, not part of the attention: the read floor of the
 * split-KV forward at the decode shape (dense keys, splits that fit LDS
 * whole).  The same workgroups as the forward's whole-chunk kernel — one per
 * 128-row tile of a batch's T*n_h rows, per batch and per split — each read
 * their rows of q (16-byte loads) and their split's K and V rows (LDS-DMA,
 * all issued at once), with no arithmetic.  out[w], one uint32 per workgroup
 * w = tile + tiles * (b + B * split), tiles = ceil(T*n_h/128), receives the
 * XOR of every 32-bit word workgroup w read (so no load can be dropped).
 *  q bf16 [B, T, n_h, hd];  k, v bf16 [B, s_k, hd];  hd in {64, 128, 256};
 *  1 <= num_splits <= s_k, and a split of ceil(s_k / num_splits) keys must fit
 *  64 KiB per tensor (else FMHA_ERR_UNSUPPORTED).  q, k, v 16-byte aligned,
 *  out 4-byte. */
int fmha_read_floor(const void* q, const void* k, const void* v, uint32_t* out,
                    int B, int T, int n_h, int s_k, int hd, int num_splits, void* stream);

/* Measurement helper, not part of the attention: the sustained rate of the
 * bf16 matrix instruction the attention kernels use (v_mfma_f32_32x32x16_bf16)
 * on given operands.  n_wg workgroups of 512 threads (eight waves; two per SIMD
 * once the chip is full) each run, per wave, `iters` rounds of four
 * independent chains D_c = A_c . B_c + D_c (c = 0..3, D_c starting at 0).
 *  ops     bf16 [8 waves][8 fragments][64 lanes][8]: fragment 2c is A_c,
 *          2c+1 is B_c, in the instruction's operand layout (lane l holds row
 *          or column l % 32 and k = 8 (l / 32) .. +7); shared by every
 *          workgroup: 65536 bytes, 16-byte aligned
 *  sums    fp32 [n_wg][8][4]: the sum of all 1024 elements of each final D_c
 *  clocks  uint64 [n_wg][2]: shader-clock cycles and 100 MHz real-time ticks
 *          wave 0 of the workgroup spent in its loop (8-byte aligned)
 * Work per launch: n_wg * 8 * 4 * iters * 32768 FLOP.  n_wg, iters >= 1. */
int fmha_mfma_ceiling(const void* ops, float* sums, uint64_t* clocks, int n_wg, int iters,
                      void* stream);

/* Log-sum-exp merge of normalised partial results (page "CURRENT ISSUE: UMMA
 * FMHA — Full Pipeline + Production", "Next steps" 4):
 *   M = max_i lse_i,  w_i = exp(lse_i - M),
 *   out = sum_i w_i o_i / sum_i w_i,  lse = M + ln sum_i w_i.
 *  o_parts    fp32 [n_parts, rows, hd], each part normalised over its keys
 *  lse_parts  fp32 [n_parts, rows], natural log; -inf marks an empty part,
 *             whose o_parts values are ignored (they may hold anything)
 *  out        [rows, hd] of out_dtype; lse fp32 [rows] (may be NULL: not written)
 * A row whose parts are all empty gets out = 0, lse = -inf.
 * n_parts >= 1, rows >= 0, hd >= 4 and a multiple of 4; o_parts and out
 * 16-byte aligned (out 8-byte for bf16). */
int fmha_lse_merge(const float* o_parts, const float* lse_parts, int n_parts,
                   int rows, int hd, void* out, int out_dtype, float* lse,
                   void* stream);

/* Index scores of the top-k indexer that produces kv_idx (the dsv4/kernels/cuda
 * commit log, indexer_score_topk: per-head scores with per-head weights, the
 * 1024 best pool entries kept per token; the formula is not printed — reading:
 * the DeepSeek sparse-attention indexer form, one index key per entry):
 *   scores[b, t, s] = sum_h w[b, t, h] * max(0, sum_c q[b, t, h, c] * k[s, c])
 *  q       bf16 [B, T, n_ih, c] index queries;  k  bf16 [P, c] index keys
 *  w       fp32 [B, T, n_ih] head weights;      scores  fp32 [B, T, P] (written)
 * n_ih in {32, 64} and c in {64, 128} (else FMHA_ERR_UNSUPPORTED); B, T >= 0;
 * P >= 1 with P*c*2 < 2^31.  q, k 16-byte aligned; w, scores 4-byte. */
int fmha_index_scores(const void* q, const void* k, const float* w, float* scores,
                      int B, int T, int n_ih, int c, int P, void* stream);

/* Exact top-k of each row of scores fp32 [rows, P] (the selection of the same
 * indexer): idx int32 [rows, top_k] receives the ids of the top_k largest
 * scores, ties broken towards the smaller id, in ascending id order; when
 * P < top_k the list is padded with -1 (a key the attention masks).
 * rows >= 0, 1 <= P <= 32768 (a row is selected in LDS; larger P gives
 * FMHA_ERR_UNSUPPORTED), top_k >= 1.  scores and idx 4-byte aligned. */
int fmha_topk_select(const float* scores, int32_t* idx, int rows, int P, int top_k,
                     void* stream);

/* Static English text for a status code (never NULL). */
const char* fmha_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FMHA_MQA_H */
