// Log-sum-exp merge of normalised partial attention outputs, for gfx950.
//
// The merge rule is the one the dev-log page "CURRENT ISSUE: UMMA FMHA — Full
// Pipeline + Production" gives under "Next steps" item 4 (Multi-KV-tile):
// parts are weighted by exp(lse_i) and the sum is divided by the sum of the
// weights.  It is evaluated shifted by the largest lse of the row so that no
// exponential overflows; the merged lse is max + ln(sum of shifted weights).
//
// The kernel is bound by HBM/L2 bandwidth: each thread owns one 16-byte chunk
// of every part's row (4 fp32 or 8 bf16 elements), reads it with 16-byte
// loads (consecutive threads -> consecutive chunks of a row, so every wave
// reads whole contiguous segments) and writes it once.  For the usual part
// counts all of a thread's loads are in flight together.
#include <math.h>

#include "fmha_device.h"

namespace fmha {
namespace {

using dev::f32x4;
using dev::u32x2;
using dev::u32x4;
using dev::pack_bf16x2;

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// NP > 0: the part count is a compile-time constant, so every lse and O load
// of a thread is issued before any arithmetic (one memory round trip per
// thread instead of one per part).  NP == 0: any count, loop over parts.
// IN_BF16: the parts hold bf16 (the split path's own partials for bf16
// outputs, whose output rows are 16-byte aligned), else fp32.  A thread owns
// one 16-byte chunk of every part's row: 8 elements of bf16 parts, 4 of fp32.
// xcd_bpg > 0: the grid has exactly one block per 256 chunks, rows come in
// groups of xcd_bpg blocks whose count is a multiple of 8, and block b takes
// the rows of a group on XCD b mod 8 (the dispatcher's order): the group whose
// splits the attention kernel ran there (1-2% faster than the plain order).
template <bool OUT_BF16, int NP, bool IN_BF16>
__global__ __launch_bounds__(256) void merge_kernel(const void* __restrict__ o_parts,
                                                    const float* __restrict__ lse_parts,
                                                    int n_parts, int rows, int hd,
                                                    void* __restrict__ out,
                                                    float* __restrict__ lse,
                                                    const float* __restrict__ sink,
                                                    int n_heads, int xcd_bpg) {
  constexpr int E = IN_BF16 ? 8 : 4;  // elements per thread
  static_assert(!IN_BF16 || OUT_BF16, "bf16 parts come with bf16 outputs");
  const int cpr = hd / E;  // chunks per row
  const int64_t total = (int64_t)rows * cpr;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int np = NP > 0 ? NP : n_parts;
  int64_t blk = blockIdx.x;
  if (xcd_bpg > 0) {
    const int x = blockIdx.x & 7, k = blockIdx.x >> 3;
    const int j = k / xcd_bpg;
    blk = (int64_t)(x + 8 * j) * xcd_bpg + (k - j * xcd_bpg);
  }
  for (int64_t u = blk * blockDim.x + threadIdx.x; u < total; u += stride) {
    const int row = (int)(u / cpr);
    const int ch = (int)(u % cpr);
    auto part = [&](int i, float (&o)[E]) __attribute__((always_inline)) {
      const int64_t off = ((int64_t)i * rows + row) * hd + E * ch;
      if constexpr (IN_BF16) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(o_parts) + off);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          o[2 * k] = __uint_as_float(w[k] << 16);
          o[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
        }
      } else {
        const f32x4 v = *reinterpret_cast<const f32x4*>(static_cast<const float*>(o_parts) + off);
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = v[k];
      }
    };
    float acc[E];
#pragma unroll
    for (int k = 0; k < E; ++k) acc[k] = 0.f;
    float mx = -__builtin_inff();
    float den = 0.f;
    if constexpr (NP > 0) {
      float li[NP];
      float oi[NP][E];
#pragma unroll
      for (int i = 0; i < NP; ++i) li[i] = lse_parts[(int64_t)i * rows + row];
#pragma unroll
      for (int i = 0; i < NP; ++i) part(i, oi[i]);
#pragma unroll
      for (int i = 0; i < NP; ++i) mx = fmaxf(mx, li[i]);
      if (mx != -__builtin_inff()) {
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          // an empty part (lse -inf) gets weight 0 and its O is not used
          const bool live = li[i] != -__builtin_inff();
          const float w = live ? __builtin_amdgcn_exp2f((li[i] - mx) * LOG2E) : 0.f;
          den += w;
          if (live) {
#pragma unroll
            for (int k = 0; k < E; ++k) acc[k] += w * oi[i][k];
          }
        }
      }
    } else {
      for (int i = 0; i < np; ++i) mx = fmaxf(mx, lse_parts[(int64_t)i * rows + row]);
      if (mx != -__builtin_inff()) {
        for (int i = 0; i < np; ++i) {
          const float li = lse_parts[(int64_t)i * rows + row];
          if (li == -__builtin_inff()) continue;  // empty part: its o_i is never read
          const float w = __builtin_amdgcn_exp2f((li - mx) * LOG2E);
          den += w;
          float oi[E];
          part(i, oi);
#pragma unroll
          for (int k = 0; k < E; ++k) acc[k] += w * oi[k];
        }
      }
    }
    float f = mx != -__builtin_inff() ? 1.f / den : 0.f;
    float lse_r = (mx != -__builtin_inff()) ? mx + log2f(den) * LN2 : -__builtin_inff();
    if (sink != nullptr) dev::sink_adjust(sink[row % n_heads], f, lse_r);
    if constexpr (OUT_BF16) {
      uint32_t w[E / 2];
#pragma unroll
      for (int k = 0; k < E / 2; ++k) w[k] = pack_bf16x2(acc[2 * k] * f, acc[2 * k + 1] * f);
      uint16_t* o = static_cast<uint16_t*>(out) + (int64_t)row * hd + E * ch;
      if constexpr (E == 8)
        *reinterpret_cast<u32x4*>(o) = u32x4{w[0], w[1], w[2], w[3]};
      else
        *reinterpret_cast<u32x2*>(o) = u32x2{w[0], w[1]};
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(out) + (int64_t)row * hd + E * ch) =
          f32x4{acc[0] * f, acc[1] * f, acc[2] * f, acc[3] * f};
    }
    if (ch == 0 && lse != nullptr) lse[row] = lse_r;
  }
}

// In-place attention sink on finished rows: one wave per row, lanes over the
// row's 16-byte chunks.  Every lane reads the row's lse before lane 0 rewrites
// it (program order within the wave), so no lane sees the updated value.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void sink_kernel(void* __restrict__ out, float* __restrict__ lse,
                                                   const float* __restrict__ sink, int rows,
                                                   int n_heads, int hd) {
  const int lane = threadIdx.x & 63;
  const int cpr = hd >> 2;
  for (int row = blockIdx.x * 4 + (threadIdx.x >> 6); row < rows; row += gridDim.x * 4) {
    float f = 1.f, l = lse[row];
    dev::sink_adjust(sink[row % n_heads], f, l);
    for (int ch = lane; ch < cpr; ch += 64) {
      if constexpr (OUT_BF16) {
        uint16_t* o = static_cast<uint16_t*>(out) + (int64_t)row * hd + 4 * ch;
        const u32x2 w = *reinterpret_cast<const u32x2*>(o);
        float x[4];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          x[2 * i] = __uint_as_float(w[i] << 16) * f;
          x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u) * f;
        }
        *reinterpret_cast<u32x2*>(o) = u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
      } else {
        f32x4* o = reinterpret_cast<f32x4*>(static_cast<float*>(out) + (int64_t)row * hd + 4 * ch);
        *o = *o * f;
      }
    }
    if (lane == 0) lse[row] = l;
  }
}

template <int NP>
void launch_np(bool out_bf16, bool parts_bf16, dim3 grid, hipStream_t stream,
               const void* o_parts, const float* lse_parts, int n_parts, int rows, int hd,
               void* out, float* lse, const float* sink, int n_heads, int xcd_bpg) {
  // bf16 parts come only with bf16 outputs
  if (parts_bf16)
    hipLaunchKernelGGL((merge_kernel<true, NP, true>), grid, dim3(256), 0, stream, o_parts,
                       lse_parts, n_parts, rows, hd, out, lse, sink, n_heads, xcd_bpg);
  else if (out_bf16)
    hipLaunchKernelGGL((merge_kernel<true, NP, false>), grid, dim3(256), 0, stream, o_parts,
                       lse_parts, n_parts, rows, hd, out, lse, sink, n_heads, xcd_bpg);
  else
    hipLaunchKernelGGL((merge_kernel<false, NP, false>), grid, dim3(256), 0, stream, o_parts,
                       lse_parts, n_parts, rows, hd, out, lse, sink, n_heads, xcd_bpg);
}

}  // namespace

hipError_t launch_merge(const void* o_parts, const float* lse_parts, int n_parts, int rows,
                        int hd, void* out, bool out_bf16, float* lse, hipStream_t stream,
                        const float* sink, int n_heads, bool parts_bf16, int group_rows) {
  const int cpr = hd / (parts_bf16 ? 8 : 4);
  const int64_t total = (int64_t)rows * cpr;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  const dim3 grid((unsigned)blocks);
  // the XCD order: whole blocks of whole rows, whole groups of blocks, a
  // multiple of 8 groups, one block per 256 chunks
  int xcd_bpg = 0;
  if (group_rows > 0 && cpr <= 256 && 256 % cpr == 0 && rows % group_rows == 0 &&
      (rows / group_rows) % 8 == 0 && group_rows % (256 / cpr) == 0 && blocks * 256 == total)
    xcd_bpg = group_rows / (256 / cpr);
  switch (n_parts) {
#define FMHA_MERGE_CASE(N) \
  case N:                  \
    launch_np<N>(out_bf16, parts_bf16, grid, stream, o_parts, lse_parts, n_parts, rows, hd, out, \
                 lse, sink, n_heads, xcd_bpg);                                                     \
    break;
    FMHA_MERGE_CASE(1) FMHA_MERGE_CASE(2) FMHA_MERGE_CASE(3) FMHA_MERGE_CASE(4)
    FMHA_MERGE_CASE(5) FMHA_MERGE_CASE(6) FMHA_MERGE_CASE(7) FMHA_MERGE_CASE(8)
    FMHA_MERGE_CASE(12) FMHA_MERGE_CASE(16)
#undef FMHA_MERGE_CASE
    default:
      launch_np<0>(out_bf16, parts_bf16, grid, stream, o_parts, lse_parts, n_parts, rows, hd, out,
                   lse, sink, n_heads, xcd_bpg);
  }
  return hipGetLastError();
}

hipError_t launch_sink(void* out, float* lse, const float* sink, int rows, int n_heads, int hd,
                       bool out_bf16, hipStream_t stream) {
  int64_t blocks = ((int64_t)rows + 3) / 4;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  if (out_bf16)
    hipLaunchKernelGGL((sink_kernel<true>), dim3((unsigned)blocks), dim3(256), 0, stream, out, lse,
                       sink, rows, n_heads, hd);
  else
    hipLaunchKernelGGL((sink_kernel<false>), dim3((unsigned)blocks), dim3(256), 0, stream, out,
                       lse, sink, rows, n_heads, hd);
  return hipGetLastError();
}

}  // namespace fmha
