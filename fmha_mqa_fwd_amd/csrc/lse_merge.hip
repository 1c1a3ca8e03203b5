// Log-sum-exp merge of normalised partial attention outputs, for gfx950.
//
// The merge rule is the one the dev-log page "CURRENT ISSUE: UMMA FMHA — Full
// Pipeline + Production" gives under "Next steps" item 4 (Multi-KV-tile):
// parts are weighted by exp(lse_i) and the sum is divided by the sum of the
// weights.  It is evaluated shifted by the largest lse of the row so that no
// exponential overflows; the merged lse is max + ln(sum of shifted weights).
//
// The kernel is bound by HBM/L2 bandwidth: each thread owns one 16-byte chunk
// (4 floats) of one output row, reads that chunk from every part with 16-byte
// loads (consecutive threads -> consecutive chunks of a row, so every wave
// reads whole contiguous segments) and writes it once.
#include <math.h>

#include "fmha_internal.h"

namespace fmha {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  __bf16 x = (__bf16)a;
  __bf16 y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) |
         ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ o_parts,
                                                    const float* __restrict__ lse_parts,
                                                    int n_parts, int rows, int hd,
                                                    void* __restrict__ out,
                                                    float* __restrict__ lse) {
  const int cpr = hd >> 2;  // 16-byte chunks per row
  const int64_t total = (int64_t)rows * cpr;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total; u += stride) {
    const int row = (int)(u / cpr);
    const int ch = (int)(u % cpr);
    float mx = -__builtin_inff();
    for (int i = 0; i < n_parts; ++i) mx = fmaxf(mx, lse_parts[(int64_t)i * rows + row]);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float den = 0.f;
    const bool live = mx != -__builtin_inff();
    if (live) {
      for (int i = 0; i < n_parts; ++i) {
        const float li = lse_parts[(int64_t)i * rows + row];
        if (li == -__builtin_inff()) continue;  // empty part: its o_i is never read
        const float w = __builtin_amdgcn_exp2f((li - mx) * LOG2E);
        den += w;
        const f32x4 oi =
            *reinterpret_cast<const f32x4*>(o_parts + ((int64_t)i * rows + row) * hd + 4 * ch);
        acc += w * oi;
      }
      acc *= 1.f / den;
    }
    if constexpr (OUT_BF16) {
      u32x2 w = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + (int64_t)row * hd + 4 * ch) = w;
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(out) + (int64_t)row * hd + 4 * ch) = acc;
    }
    if (ch == 0 && lse != nullptr) lse[row] = live ? mx + log2f(den) * LN2 : -__builtin_inff();
  }
}

}  // namespace

hipError_t launch_merge(const float* o_parts, const float* lse_parts, int n_parts, int rows,
                        int hd, void* out, bool out_bf16, float* lse, hipStream_t stream) {
  const int64_t total = (int64_t)rows * (hd / 4);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  if (out_bf16)
    hipLaunchKernelGGL(merge_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, o_parts,
                       lse_parts, n_parts, rows, hd, out, lse);
  else
    hipLaunchKernelGGL(merge_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, o_parts,
                       lse_parts, n_parts, rows, hd, out, lse);
  return hipGetLastError();
}

}  // namespace fmha
