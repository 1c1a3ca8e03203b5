// C ABI of libfmha_mqa.so: argument validation, work decomposition and
// launches.  Declarations and the contract live in include/fmha_mqa.h.
//
// Every function validates all arguments before it enqueues anything, never
// allocates, frees or synchronises, and reports errors as status codes.  The
// compile-once / launch-many shape and the absence of host syncs follow the
// lessons in the dsv4/kernels/cuda commit log (per-call JIT and .item() syncs
// dominated the time there).
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "fmha_internal.h"
#include "fmha_mqa.h"

// Scratch memory of fmha_mqa_fwd_noalloc: the split-KV workspace for callers
// that cannot allocate.  Each GPU the library runs on holds its own copy for
// the life of the process.  In host code `scratch` names a host-side stand-in,
// never the device memory: kernels and copies use the per-device address that
// hipGetSymbolAddress returns (scratch_address below).
static __device__ __align__(256) char scratch[FMHA_SCRATCH_BYTES];

namespace {

constexpr size_t kRegionAlign = 256;

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline bool aligned(const void* p, size_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

// Workspace layout for split-KV: o_part fp32 [S, rows, hd], then lse_part fp32 [S, rows].
struct WsLayout {
  size_t o_bytes, lse_off, total;
};

inline WsLayout ws_layout(int64_t rows, int hd, int splits) {
  WsLayout w;
  w.o_bytes = round_up((size_t)splits * (size_t)rows * (size_t)hd * 4u, kRegionAlign);
  w.lse_off = w.o_bytes;
  w.total = w.o_bytes + round_up((size_t)splits * (size_t)rows * 4u, kRegionAlign);
  return w;
}

inline int launch_status(hipError_t e) { return e == hipSuccess ? FMHA_OK : FMHA_ERR_LAUNCH; }

// The forward of fmha_mqa_fwd / fmha_mqa_fwd_sink (sink: nullptr or [n_h]),
// and, with partials_only, of fmha_mqa_fwd_partials: out/lse are then the
// caller's fp32 partial planes [num_splits, rows, hd] / [num_splits, rows],
// written without a merge (out_dtype, sink and workspace unused).
// validate_only: return the validation status without launching anything
// (the workspace is not looked at).
int fwd_impl(const void* q, const void* k, const void* v, const int32_t* kv_idx, void* out,
             float* lse, int B, int T, int n_h, int s_k, int hd, int pool_rows, float scale,
             int out_dtype, int num_splits, void* workspace, size_t workspace_bytes,
             void* stream, const float* sink, bool partials_only = false,
             bool validate_only = false) {
  if (out_dtype != FMHA_F32 && out_dtype != FMHA_BF16) return FMHA_ERR_INVALID_ARG;
  if (B < 0 || T < 0 || n_h < 0 || s_k < 0 || num_splits < 1) return FMHA_ERR_INVALID_ARG;
  if (hd != 64 && hd != 128 && hd != 256 && hd != 512) return FMHA_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || !isfinite(scale)) return FMHA_ERR_INVALID_ARG;
  const int64_t rows = (int64_t)B * T * n_h;
  if (rows == 0) return FMHA_OK;  // nothing to compute
  if (rows > INT32_MAX) return FMHA_ERR_UNSUPPORTED;
  if (num_splits > (s_k > 1 ? s_k : 1)) return FMHA_ERR_INVALID_ARG;
  if (!q || !out || !lse) return FMHA_ERR_INVALID_ARG;
  const bool gather = kv_idx != nullptr;
  if (s_k > 0) {
    if (!k || !v) return FMHA_ERR_INVALID_ARG;
    if (gather && pool_rows < 1) return FMHA_ERR_INVALID_ARG;
    // K/V rows are addressed with 32-bit byte offsets per batch (dense) or
    // per pool (gather)
    const int64_t kv_rows = gather ? (int64_t)pool_rows : (int64_t)s_k;
    if (kv_rows * hd * 2 > INT32_MAX) return FMHA_ERR_UNSUPPORTED;
  }
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(lse, 4)) return FMHA_ERR_ALIGNMENT;
  if (s_k > 0 && (!aligned(k, 16) || !aligned(v, 16))) return FMHA_ERR_ALIGNMENT;
  if (gather && !aligned(kv_idx, 4)) return FMHA_ERR_ALIGNMENT;
  if (sink && !aligned(sink, 4)) return FMHA_ERR_ALIGNMENT;

  fmha::FwdParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.kv_idx = (gather && s_k > 0) ? kv_idx : nullptr;
  p.total_rows = rows;
  p.rows_per_group = gather ? n_h : T * n_h;
  p.n_groups = gather ? B * T : B;
  p.s_k = s_k;
  p.pool_rows = gather ? pool_rows : 0;
  p.num_splits = num_splits;
  p.chunk = (s_k + num_splits - 1) / num_splits;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.sink = sink;
  p.n_heads = n_h;
  if (gather && s_k == 0) p.n_groups = B * T;  // still one group per token

  const int64_t grid = fmha::fwd_grid_size(p, hd);
  if (grid > INT32_MAX) return FMHA_ERR_UNSUPPORTED;
  if (validate_only) return FMHA_OK;

  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // launch errors below are ours alone

  if (partials_only) {
    p.out = out;
    p.lse = lse;
    p.out_mode = fmha::OUT_PARTIAL;
    return launch_status(fmha::launch_fwd(p, hd, st));
  }
  if (num_splits == 1) {
    p.out = out;
    p.lse = lse;
    p.out_mode = out_dtype == FMHA_BF16 ? fmha::OUT_BF16 : fmha::OUT_F32;
    return launch_status(fmha::launch_fwd(p, hd, st));
  }

  const WsLayout wl = ws_layout(rows, hd, num_splits);
  if (!workspace || !aligned(workspace, 16) || workspace_bytes < wl.total)
    return FMHA_ERR_WORKSPACE;
  // bf16 outputs keep bf16 partials (their rounding is of the output's own
  // order; the partial traffic halves); fp32 outputs keep fp32 partials
  const bool bf16_parts = out_dtype == FMHA_BF16;
  void* o_part = workspace;
  float* lse_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + wl.lse_off);
  p.out = o_part;
  p.lse = lse_part;
  p.out_mode = bf16_parts ? fmha::OUT_PARTIAL_BF16 : fmha::OUT_PARTIAL;
  int s = launch_status(fmha::launch_fwd(p, hd, st));
  if (s != FMHA_OK) return s;
  // the sink joins once, in the merge (the partials carry none).  With a
  // multiple of 8 groups of at most 512 rows (at most 8 row tiles), the
  // attention kernels' placement put every split and tile of group g on XCD
  // g mod 8 (wg_coords), and the merge follows it.
  const int group_rows = (p.n_groups % 8 == 0 && p.rows_per_group <= 512) ? p.rows_per_group : 0;
  return launch_status(fmha::launch_merge(o_part, lse_part, num_splits, (int)rows, hd, out,
                                          out_dtype == FMHA_BF16, lse, st, sink, n_h,
                                          bf16_parts, group_rows));
}

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The device address of `scratch` on the GPU that runs `stream`, looked up
// once per device with that device current.  nullptr if the lookup failed.
void* scratch_address(hipStream_t stream) {
  int dev = -1;
  if (stream != nullptr) {
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return nullptr;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_scratch_once[dev], [dev]() {
    int prev = -1;
    g_scratch_err[dev] = hipGetDevice(&prev);
    if (g_scratch_err[dev] != hipSuccess) return;
    if (prev != dev) g_scratch_err[dev] = hipSetDevice(dev);
    void* ptr = nullptr;
    if (g_scratch_err[dev] == hipSuccess)
      g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (g_scratch_err[dev] == hipSuccess) g_scratch_ptr[dev] = ptr;
    if (prev != dev) (void)hipSetDevice(prev);
  });
  return g_scratch_err[dev] == hipSuccess ? g_scratch_ptr[dev] : nullptr;
}

}  // namespace

extern "C" {

size_t fmha_mqa_workspace_bytes(int B, int T, int n_h, int hd, int num_splits) {
  if (B < 0 || T < 0 || n_h < 0 || hd <= 0 || num_splits < 1) return 0;
  if (num_splits == 1) return 0;
  const int64_t rows = (int64_t)B * T * n_h;
  return ws_layout(rows, hd, num_splits).total;
}

int fmha_mqa_fwd(const void* q, const void* k, const void* v, const int32_t* kv_idx, void* out,
                 float* lse, int B, int T, int n_h, int s_k, int hd, int pool_rows, float scale,
                 int out_dtype, int num_splits, void* workspace, size_t workspace_bytes,
                 void* stream) {
  return fwd_impl(q, k, v, kv_idx, out, lse, B, T, n_h, s_k, hd, pool_rows, scale, out_dtype,
                  num_splits, workspace, workspace_bytes, stream, nullptr);
}

int fmha_mqa_fwd_sink(const void* q, const void* k, const void* v, const int32_t* kv_idx,
                      void* out, float* lse, int B, int T, int n_h, int s_k, int hd, int pool_rows,
                      float scale, int out_dtype, int num_splits, void* workspace,
                      size_t workspace_bytes, void* stream, const float* sink) {
  if (!sink) return FMHA_ERR_INVALID_ARG;
  return fwd_impl(q, k, v, kv_idx, out, lse, B, T, n_h, s_k, hd, pool_rows, scale, out_dtype,
                  num_splits, workspace, workspace_bytes, stream, sink);
}

int fmha_mqa_fwd_noalloc(const void* q, const void* k, const void* v, const int32_t* kv_idx,
                         void* out, float* lse, int B, int T, int n_h, int s_k, int hd,
                         int pool_rows, float scale, int out_dtype, int num_splits,
                         void* stream) {
  // every argument is checked before the device is touched
  const int s = fwd_impl(q, k, v, kv_idx, out, lse, B, T, n_h, s_k, hd, pool_rows, scale,
                         out_dtype, num_splits, nullptr, 0, stream, nullptr, false, true);
  if (s != FMHA_OK) return s;
  void* ws = nullptr;
  const int64_t rows = (int64_t)B * T * n_h;
  if (num_splits > 1 && rows > 0) {
    if (ws_layout(rows, hd, num_splits).total > (size_t)FMHA_SCRATCH_BYTES)
      return FMHA_ERR_SCRATCH_LIMIT;
    ws = scratch_address(static_cast<hipStream_t>(stream));
    if (ws == nullptr) return FMHA_ERR_LAUNCH;
  }
  return fwd_impl(q, k, v, kv_idx, out, lse, B, T, n_h, s_k, hd, pool_rows, scale, out_dtype,
                  num_splits, ws, ws ? (size_t)FMHA_SCRATCH_BYTES : 0, stream, nullptr);
}

int fmha_mqa_fwd_partials(const void* q, const void* k, const void* v, const int32_t* kv_idx,
                          float* o_parts, float* lse_parts, int B, int T, int n_h, int s_k,
                          int hd, int pool_rows, float scale, int num_splits, void* stream) {
  return fwd_impl(q, k, v, kv_idx, o_parts, lse_parts, B, T, n_h, s_k, hd, pool_rows, scale,
                  FMHA_F32, num_splits, nullptr, 0, stream, nullptr, true);
}

int fmha_mqa_fwd_sources_partials(const void* q, const fmha_kv_source* sources, int n_sources,
                                  float* o_parts, float* lse_parts, int B, int T, int n_h,
                                  int hd, float scale, void* stream) {
  if (n_sources < 1 || !sources) return FMHA_ERR_INVALID_ARG;
  // every source is checked before anything is launched
  bool fused = hd == 512 && n_sources <= fmha::MAX_SOURCES;
  for (int i = 0; i < n_sources; ++i) {
    const fmha_kv_source& s = sources[i];
    const int st = fwd_impl(q, s.k, s.v, s.kv_idx, o_parts, lse_parts, B, T, n_h, s.s_k, hd,
                            s.pool_rows, scale, FMHA_F32, s.num_splits, nullptr, 0, stream,
                            nullptr, true, true);
    if (st != FMHA_OK) return st;
    const int chunk = (s.s_k + s.num_splits - 1) / s.num_splits;
    if (chunk > fmha::fwd512_max_keys()) fused = false;
  }
  const int64_t rows = (int64_t)B * T * n_h;
  if (rows == 0) return FMHA_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (!fused) {
    // one launch per source, each into its own planes
    int64_t plane = 0;
    for (int i = 0; i < n_sources; ++i) {
      const fmha_kv_source& s = sources[i];
      const int r = fwd_impl(q, s.k, s.v, s.kv_idx, o_parts + plane * rows * hd,
                             lse_parts + plane * rows, B, T, n_h, s.s_k, hd, s.pool_rows,
                             scale, FMHA_F32, s.num_splits, nullptr, 0, stream, nullptr, true);
      if (r != FMHA_OK) return r;
      plane += s.num_splits;
    }
    return FMHA_OK;
  }
  // one launch: each source laid out as its own fmha_mqa_fwd_partials would be
  fmha::SourcesParams sp{};
  sp.base.q = static_cast<const uint16_t*>(q);
  sp.base.out = o_parts;
  sp.base.lse = lse_parts;
  sp.base.total_rows = rows;
  sp.base.out_mode = fmha::OUT_PARTIAL;
  sp.base.scale_log2 = scale * 1.4426950408889634f;
  sp.base.n_heads = n_h;
  sp.n_src = n_sources;
  int plane = 0;
  int64_t grid = 0;
  for (int i = 0; i < n_sources; ++i) {
    const fmha_kv_source& s = sources[i];
    const bool gather = s.kv_idx != nullptr;
    fmha::SourceParams& d = sp.src[i];
    d.k = static_cast<const uint16_t*>(s.k);
    d.v = static_cast<const uint16_t*>(s.v);
    d.kv_idx = (gather && s.s_k > 0) ? s.kv_idx : nullptr;
    d.s_k = s.s_k;
    d.pool_rows = gather ? s.pool_rows : 0;
    d.num_splits = s.num_splits;
    d.chunk = (s.s_k + s.num_splits - 1) / s.num_splits;
    d.n_groups = gather ? B * T : B;
    d.rows_per_group = gather ? n_h : T * n_h;
    d.plane_begin = plane;
    plane += s.num_splits;
    grid += (int64_t)((d.rows_per_group + 63) / 64) * d.n_groups * d.num_splits;
  }
  if (grid > INT32_MAX) return FMHA_ERR_UNSUPPORTED;
  (void)hipGetLastError();  // launch errors below are ours alone
  return launch_status(fmha::launch_fwd512_sources(sp, st));
}

int fmha_attention_sink(void* out, float* lse, const float* sink, int rows, int n_h, int hd,
                        int out_dtype, void* stream) {
  if (out_dtype != FMHA_F32 && out_dtype != FMHA_BF16) return FMHA_ERR_INVALID_ARG;
  if (rows < 0 || n_h < 1 || hd < 4 || (hd % 4) != 0) return FMHA_ERR_INVALID_ARG;
  if (rows == 0) return FMHA_OK;
  if (!out || !lse || !sink) return FMHA_ERR_INVALID_ARG;
  if (!aligned(out, out_dtype == FMHA_BF16 ? 8 : 16) || !aligned(lse, 4) || !aligned(sink, 4))
    return FMHA_ERR_ALIGNMENT;
  (void)hipGetLastError();
  return launch_status(fmha::launch_sink(out, lse, sink, rows, n_h, hd, out_dtype == FMHA_BF16,
                                         static_cast<hipStream_t>(stream)));
}

int fmha_index_scores(const void* q, const void* k, const float* w, float* scores, int B, int T,
                      int n_ih, int c, int P, void* stream) {
  if (B < 0 || T < 0 || P < 1) return FMHA_ERR_INVALID_ARG;
  if ((n_ih != 32 && n_ih != 64) || (c != 64 && c != 128)) return FMHA_ERR_UNSUPPORTED;
  const int64_t tokens = (int64_t)B * T;
  if (tokens == 0) return FMHA_OK;
  if (tokens > INT32_MAX || (int64_t)P * c * 2 > INT32_MAX) return FMHA_ERR_UNSUPPORTED;
  if (!q || !k || !w || !scores) return FMHA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(w, 4) || !aligned(scores, 4))
    return FMHA_ERR_ALIGNMENT;
  (void)hipGetLastError();
  return launch_status(fmha::launch_index_scores(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), w, scores, (int)tokens,
      n_ih, c, P, static_cast<hipStream_t>(stream)));
}

int fmha_topk_select(const float* scores, int32_t* idx, int rows, int P, int top_k,
                     void* stream) {
  if (rows < 0 || P < 1 || top_k < 1) return FMHA_ERR_INVALID_ARG;
  if (P > fmha::topk_max_pool()) return FMHA_ERR_UNSUPPORTED;
  if (rows == 0) return FMHA_OK;
  if (!scores || !idx) return FMHA_ERR_INVALID_ARG;
  if (!aligned(scores, 4) || !aligned(idx, 4)) return FMHA_ERR_ALIGNMENT;
  (void)hipGetLastError();
  return launch_status(
      fmha::launch_topk(scores, idx, rows, P, top_k, static_cast<hipStream_t>(stream)));
}

int fmha_gather_floor(const void* k, const void* v, const int32_t* kv_idx, uint32_t* out,
                      int B, int T, int s_k, int hd, int pool_rows, void* stream) {
  if (B < 0 || T < 0 || s_k < 0 || pool_rows < 1) return FMHA_ERR_INVALID_ARG;
  if (hd != 64 && hd != 128 && hd != 256 && hd != 512) return FMHA_ERR_UNSUPPORTED;
  const int64_t tokens = (int64_t)B * T;
  if (tokens == 0) return FMHA_OK;
  if (tokens > INT32_MAX || (int64_t)pool_rows * hd * 2 > INT32_MAX ||
      (int64_t)s_k * hd * 2 / 16 > INT32_MAX)
    return FMHA_ERR_UNSUPPORTED;
  if (!k || !v || !kv_idx || !out) return FMHA_ERR_INVALID_ARG;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(kv_idx, 4) || !aligned(out, 4))
    return FMHA_ERR_ALIGNMENT;
  (void)hipGetLastError();
  return launch_status(fmha::launch_gather_floor(
      static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), kv_idx, out, (int)tokens,
      s_k, hd, pool_rows, static_cast<hipStream_t>(stream)));
}

int fmha_read_floor(const void* q, const void* k, const void* v, uint32_t* out, int B, int T,
                    int n_h, int s_k, int hd, int num_splits, void* stream) {
  if (B < 0 || T < 0 || n_h < 0 || s_k < 1 || num_splits < 1 || num_splits > s_k)
    return FMHA_ERR_INVALID_ARG;
  if (hd != 64 && hd != 128 && hd != 256) return FMHA_ERR_UNSUPPORTED;
  const int64_t rows = (int64_t)B * T * n_h;
  if (rows == 0) return FMHA_OK;
  const int chunk = (s_k + num_splits - 1) / num_splits;
  if (chunk > fmha::read_floor_max_keys(hd) || (int64_t)T * n_h > INT32_MAX ||
      (int64_t)s_k * hd * 2 > INT32_MAX)
    return FMHA_ERR_UNSUPPORTED;
  const int64_t grid = ((int64_t)T * n_h + 127) / 128 * B * num_splits;
  if (grid > INT32_MAX) return FMHA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !out) return FMHA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 4))
    return FMHA_ERR_ALIGNMENT;
  (void)hipGetLastError();
  return launch_status(fmha::launch_read_floor(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), out, hd, T * n_h, B, s_k, num_splits,
      static_cast<hipStream_t>(stream)));
}

int fmha_mfma_ceiling(const void* ops, float* sums, uint64_t* clocks, int n_wg, int iters,
                      void* stream) {
  if (n_wg < 1 || iters < 1) return FMHA_ERR_INVALID_ARG;
  if (!ops || !sums || !clocks) return FMHA_ERR_INVALID_ARG;
  if (!aligned(ops, 16) || !aligned(sums, 4) || !aligned(clocks, 8)) return FMHA_ERR_ALIGNMENT;
  (void)hipGetLastError();
  return launch_status(fmha::launch_mfma_ceiling(ops, sums, clocks, n_wg, iters,
                                                 static_cast<hipStream_t>(stream)));
}

int fmha_lse_merge(const float* o_parts, const float* lse_parts, int n_parts, int rows, int hd,
                   void* out, int out_dtype, float* lse, void* stream) {
  if (out_dtype != FMHA_F32 && out_dtype != FMHA_BF16) return FMHA_ERR_INVALID_ARG;
  if (n_parts < 1 || rows < 0 || hd < 4 || (hd % 4) != 0) return FMHA_ERR_INVALID_ARG;
  if (rows == 0) return FMHA_OK;
  if (!o_parts || !lse_parts || !out) return FMHA_ERR_INVALID_ARG;
  if ((int64_t)n_parts * rows * hd > (INT64_MAX / 8)) return FMHA_ERR_UNSUPPORTED;
  if (!aligned(o_parts, 16) || !aligned(lse_parts, 4)) return FMHA_ERR_ALIGNMENT;
  if (!aligned(out, out_dtype == FMHA_BF16 ? 8 : 16)) return FMHA_ERR_ALIGNMENT;
  if (lse && !aligned(lse, 4)) return FMHA_ERR_ALIGNMENT;
  (void)hipGetLastError();
  return launch_status(fmha::launch_merge(o_parts, lse_parts, n_parts, rows, hd, out,
                                          out_dtype == FMHA_BF16, lse,
                                          static_cast<hipStream_t>(stream)));
}

const char* fmha_status_string(int status) {
  switch (status) {
    case FMHA_OK: return "ok";
    case FMHA_ERR_INVALID_ARG: return "invalid argument";
    case FMHA_ERR_UNSUPPORTED: return "unsupported head dim or size";
    case FMHA_ERR_ALIGNMENT: return "misaligned pointer";
    case FMHA_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case FMHA_ERR_LAUNCH: return "kernel launch failed";
    case FMHA_ERR_SCRATCH_LIMIT:
      return "split-KV partials exceed the static scratch buffer (FMHA_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

}  // extern "C"
