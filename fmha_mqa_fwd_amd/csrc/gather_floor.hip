// Gather-only floor for the top-k row gather: the bytes the sparse attention
// must move (every gathered K and V row of every token), read with the same
// row-per-16-lanes 16-byte pattern and no attention arithmetic.  Its time is
// the memory side's floor for that access pattern; the attention kernel's
// time beside it says how much the compute adds.  A list of up to
// FLOOR_STAGED keys is read in the pool-region order the attention kernels
// walk it in (order_by_region), longer lists in list order.  Each token's
// rows are folded into one XOR word so that no load can be dropped (the word
// does not depend on the order).
#include "fmha_device.h"

namespace fmha {
namespace {

using dev::u32x4;

constexpr int FLOOR_THREADS = 256;
constexpr int FLOOR_UNROLL = 8;  // loads in flight per thread
constexpr int FLOOR_STAGED = 1024;  // longest list staged in LDS in region order

template <int HD>
__global__ __launch_bounds__(FLOOR_THREADS) void gather_floor_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ kv_idx, uint32_t* __restrict__ out, int s_k, int pool_rows) {
  constexpr int ROW = HD * 2;      // bytes per row
  constexpr int CPR = ROW / 16;    // 16-byte chunks per row
  const int64_t token = blockIdx.x;
  const int32_t* idx = kv_idx + token * s_k;
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc((void*)k, (short)0, pool_rows * ROW, dev::BUF_FLAGS);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc((void*)v, (short)0, pool_rows * ROW, dev::BUF_FLAGS);
  const int total = s_k * CPR;     // chunks of K (and as many of V)
  __shared__ uint32_t sRow[FLOOR_STAGED];  // the list as pool byte offsets, region order
  __shared__ int sCnt[FLOOR_STAGED];       // the sort's scratch
  const bool staged = s_k <= FLOOR_STAGED;
  if (staged) {
    constexpr int SLOTS = FLOOR_STAGED / FLOOR_THREADS;
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int sh = dev::region_shift(pool_rows);
    uint32_t offv[SLOTS];
    int cls[SLOTS];
#pragma unroll
    for (int e = 0; e < SLOTS; ++e) {
      const int i = tid + FLOOR_THREADS * e;
      const int r = i < s_k ? idx[i] : -1;
      const bool ok = r >= 0 && r < pool_rows;
      offv[e] = ok ? (uint32_t)r * ROW : dev::OOB;
      cls[e] = ok ? r >> sh : dev::REGION_NONE;
    }
    dev::order_by_region<FLOOR_THREADS / 64, SLOTS>(offv, cls, s_k, sRow, sCnt, wave, tid & 63);
    __syncthreads();
  }
  uint32_t acc = 0;
  for (int base = threadIdx.x; base < total; base += FLOOR_THREADS * FLOOR_UNROLL) {
    u32x4 x[2 * FLOOR_UNROLL];
#pragma unroll
    for (int u = 0; u < FLOOR_UNROLL; ++u) {
      const int c = base + u * FLOOR_THREADS;
      uint32_t off = dev::OOB;  // beyond the descriptor: reads zeros
      if (c < total) {
        if (staged) {
          const uint32_t ro = sRow[c / CPR];
          if (ro != dev::OOB) off = ro + 16u * (c % CPR);
        } else {
          const int r = idx[c / CPR];
          if (r >= 0 && r < pool_rows) off = (uint32_t)r * ROW + 16u * (c % CPR);
        }
      }
      x[2 * u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
      x[2 * u + 1] =
          __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0));
    }
#pragma unroll
    for (int u = 0; u < 2 * FLOOR_UNROLL; ++u) acc ^= x[u][0] ^ x[u][1] ^ x[u][2] ^ x[u][3];
  }
  // workgroup XOR: waves through shuffles, then LDS
  for (int d = 32; d >= 1; d >>= 1) acc ^= __shfl_xor(acc, d);
  __shared__ uint32_t part[FLOOR_THREADS / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int w = 0; w < FLOOR_THREADS / 64; ++w) r ^= part[w];
    out[token] = r;
  }
}

template <int HD>
hipError_t launch_floor_t(const uint16_t* k, const uint16_t* v, const int32_t* idx,
                          uint32_t* out, int tokens, int s_k, int pool_rows, hipStream_t st) {
  hipLaunchKernelGGL((gather_floor_kernel<HD>), dim3(tokens), dim3(FLOOR_THREADS), 0, st, k, v,
                     idx, out, s_k, pool_rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gather_floor(const uint16_t* k, const uint16_t* v, const int32_t* idx,
                               uint32_t* out, int tokens, int s_k, int hd, int pool_rows,
                               hipStream_t st) {
  switch (hd) {
    case 64: return launch_floor_t<64>(k, v, idx, out, tokens, s_k, pool_rows, st);
    case 128: return launch_floor_t<128>(k, v, idx, out, tokens, s_k, pool_rows, st);
    case 256: return launch_floor_t<256>(k, v, idx, out, tokens, s_k, pool_rows, st);
    case 512: return launch_floor_t<512>(k, v, idx, out, tokens, s_k, pool_rows, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fmha
