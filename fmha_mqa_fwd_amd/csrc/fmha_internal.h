// Internal interface between the C-ABI layer (api.hip) and the kernels.
// Not installed; callers use include/fmha_mqa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fmha {

// OUT_PARTIAL(_BF16): split partials, normalised O as fp32 (bf16) in plane
// `split` of [num_splits, total_rows, hd], lse fp32 [num_splits, total_rows].
enum OutMode : int { OUT_F32 = 0, OUT_BF16 = 1, OUT_PARTIAL = 2, OUT_PARTIAL_BF16 = 3 };

__host__ __device__ inline bool is_partial(int mode) {
  return mode == OUT_PARTIAL || mode == OUT_PARTIAL_BF16;
}
__host__ __device__ inline bool is_bf16(int mode) {
  return mode == OUT_BF16 || mode == OUT_PARTIAL_BF16;
}

// One launch of the attention kernel.  Rows r = (b*T + t)*n_h + h of q/out are
// split into groups that share one K/V set: a batch (dense, T*n_h rows) or a
// token (gather, n_h rows).  Row r belongs to group r / rows_per_group.
struct FwdParams {
  const uint16_t* q;        // bf16 [total_rows, hd]
  const uint16_t* k;        // bf16 [n_groups, s_k, hd] (dense) or [pool_rows, hd]
  const uint16_t* v;        // same layout as k
  const int32_t* kv_idx;    // gather: int32 [n_groups, s_k]; dense: nullptr
  void* out;                // OUT_F32/OUT_BF16: [total_rows, hd];
                            // partial modes: [num_splits, total_rows, hd]
  float* lse;               // [total_rows] or, partial, [num_splits, total_rows]
  int64_t total_rows;
  int rows_per_group;
  int n_groups;
  int tiles_per_group;      // filled in by launch_fwd for the chosen tile shape
  int s_k;
  int pool_rows;
  int chunk;                // keys per split (== s_k when unsplit)
  int num_splits;
  int out_mode;             // OutMode
  float scale_log2;         // softmax scale * log2(e)
  const float* sink;        // optional [n_heads] sink logits (ln units); applied by
                            // the epilogue of OUT_F32/OUT_BF16 launches only
  int n_heads;              // head of global row g is g % n_heads
};

// Picks the tile shape for hd / rows_per_group, sets p.tiles_per_group and
// launches on `stream`.  Returns the launch status.
hipError_t launch_fwd(FwdParams p, int hd, hipStream_t stream);

// Number of workgroups launch_fwd would start (for the host-side size check).
int64_t fwd_grid_size(const FwdParams& p, int hd);

// Whole-chunk variant: valid when one split's keys (p.chunk) number at most
// chunk_max_keys(hd); stages them in LDS at once.  Sets p.tiles_per_group.
int chunk_max_keys(int hd);
hipError_t launch_chunk(FwdParams p, int hd, hipStream_t stream);

// fmha_hd512.hip: head dim 512, gather or dense, for splits of at most
// fwd512_max_keys() keys (p.tiles_per_group set for 64-row tiles).
int fwd512_max_keys();
hipError_t launch_fwd512(const FwdParams& p, hipStream_t stream);

// Several key sources in one head-dim-512 launch, partial mode: source i's
// splits write planes plane_begin .. plane_begin + num_splits - 1 of the
// launch's [sum of splits, total_rows, hd] buffer (base.out / base.lse).
// Each source is laid out as a one-source launch would be (its groups: a
// token when it gathers, a batch when dense); launch_fwd512_sources fills in
// tiles_per_group and wg_begin.  Every source's chunk is at most
// fwd512_max_keys().
constexpr int MAX_SOURCES = 4;
struct SourceParams {
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* kv_idx;  // nullptr: dense
  int s_k, pool_rows, chunk, num_splits, n_groups, rows_per_group, tiles_per_group;
  int wg_begin;           // first workgroup of this source
  int plane_begin;        // first partial plane of this source
};
struct SourcesParams {
  FwdParams base;         // q, out, lse, total_rows, out_mode, scale_log2, n_heads
  int n_src;
  SourceParams src[MAX_SOURCES];
};
hipError_t launch_fwd512_sources(SourcesParams sp, hipStream_t stream);

// out[r] = sum_i w_i o_i[r] / sum_i w_i with w_i = exp(lse_i[r] - max_i lse_i[r]).
// o_parts holds fp32, or bf16 when parts_bf16.  With sink (optional,
// [n_heads]), the sink of row r's head r % n_heads joins the merged result
// (see sink_adjust in fmha_device.h).  group_rows > 0: the parts were written
// by a launch whose every split and row tile of group g (group_rows rows) ran
// on XCD g mod 8; the merge then takes each group's rows on that XCD.
hipError_t launch_merge(const void* o_parts, const float* lse_parts, int n_parts,
                        int rows, int hd, void* out, bool out_bf16, float* lse,
                        hipStream_t stream, const float* sink = nullptr, int n_heads = 1,
                        bool parts_bf16 = false, int group_rows = 0);

// In place: out[r] *= exp(lse[r] - lse'[r]), lse'[r] = ln(exp(lse[r]) + exp(sink[r % n_heads])).
hipError_t launch_sink(void* out, float* lse, const float* sink, int rows, int n_heads, int hd,
                       bool out_bf16, hipStream_t stream);

// Top-k indexer: scores [tokens, P] fp32 from q bf16 [tokens, H, C], k bf16
// [P, C], w fp32 [tokens, H] (H in {32, 64}, C in {64, 128}); selection of the
// top_k largest scores of each row (P <= topk_max_pool()) into idx int32
// [rows, top_k], ascending entry ids, -1 padding.
hipError_t launch_index_scores(const uint16_t* q, const uint16_t* k, const float* w,
                               float* scores, int tokens, int H, int C, int P,
                               hipStream_t stream);
int topk_max_pool();
// gather_floor.hip: every gathered K and V row read once, no arithmetic
hipError_t launch_gather_floor(const uint16_t* k, const uint16_t* v, const int32_t* idx,
                               uint32_t* out, int tokens, int s_k, int hd, int pool_rows,
                               hipStream_t stream);
hipError_t launch_topk(const float* scores, int32_t* idx, int rows, int P, int top_k,
                       hipStream_t stream);
// measure.hip: the whole-chunk kernel's reads with no arithmetic (dense
// groups of rows_per_group rows; chunk of ceil(s_k / num_splits) keys, at most
// read_floor_max_keys(hd)), and the sustained bf16 MFMA rate
int read_floor_max_keys(int hd);
hipError_t launch_read_floor(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             uint32_t* out, int hd, int rows_per_group, int n_groups, int s_k,
                             int num_splits, hipStream_t stream);
hipError_t launch_mfma_ceiling(const void* ops, float* sums, uint64_t* clocks, int n_wg,
                               int iters, hipStream_t stream);

}  // namespace fmha
