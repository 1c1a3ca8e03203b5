// Measurement helpers (not part of the attention): ceilings that the
// attention kernels' rates are compared with.
//
//   * read_floor_kernel — the data movement of the whole-chunk split-KV kernel
//     (fmha_chunk.hip) with no arithmetic: the same grid (128-row tiles x
//     groups x splits) and, per workgroup, the same bytes: its rows of q by
//     plain 16-byte loads, its split's K and V rows into LDS by LDS-DMA, all
//     issued at once.  Every word is folded into an XOR so that no load can be
//     dropped.  Its time is the floor of the decode split kernel's reads.
//   * mfma_kernel — the sustained rate of v_mfma_f32_32x32x16_bf16, the
//     instruction the attention kernels contract with, on given operands (the
//     matrix units draw more power on random data than on zeros, and the clock
//     follows): four independent accumulator chains per wave, two waves per
//     SIMD, shader and real-time clock read in the kernel.
#include "fmha_device.h"

namespace fmha {
namespace {

using namespace dev;

constexpr int FLOOR_TENSOR_BYTES = 64 * 1024;  // per tensor: the whole-chunk kernel's chunk

__global__ __launch_bounds__(256) void read_floor_kernel(const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v,
                                                         uint32_t* __restrict__ out, int hd,
                                                         int rows_per_group, int n_groups,
                                                         int tiles_per_group, int s_k, int chunk) {
  __shared__ __attribute__((aligned(1024))) char sK[FLOOR_TENSOR_BYTES];
  __shared__ __attribute__((aligned(1024))) char sV[FLOOR_TENSOR_BYTES];
  __shared__ uint32_t sPart[4];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int bid = blockIdx.x;
  const int tile = bid % tiles_per_group;
  bid /= tiles_per_group;
  const int group = bid % n_groups;
  const int split = bid / n_groups;
  const int key_lo = min(split * chunk, s_k);
  const int nk = min(key_lo + chunk, s_k) - key_lo;
  const int row_bytes = hd * 2;
  const int bytes = nk * row_bytes;  // <= FLOOR_TENSOR_BYTES (host guarantees)
  const int64_t kv_base = ((int64_t)group * s_k + key_lo) * hd;
  const u32x4 rk = buffer_rsrc(k + kv_base, (uint32_t)bytes);
  const u32x4 rv = buffer_rsrc(v + kv_base, (uint32_t)bytes);
  // K and V: one 1 KiB DMA instruction per KiB, spread over the four waves
  const int n_inst = (bytes + 1023) / 1024;
  for (int i = wave; i < n_inst; i += 4) {
    dma16(rk, (uint32_t)(uintptr_t)(sK + i * 1024), (uint32_t)(i * 1024 + lane * 16));
    dma16(rv, (uint32_t)(uintptr_t)(sV + i * 1024), (uint32_t)(i * 1024 + lane * 16));
  }
  // q: the workgroup's rows (at most 128), 16 bytes per load
  const int r0 = tile * 128;
  const int rows = min(128, rows_per_group - r0);
  const u32x4* qb = reinterpret_cast<const u32x4*>(q + ((int64_t)group * rows_per_group + r0) * hd);
  const int q_chunks = rows * row_bytes / 16;
  uint32_t acc = 0;
  for (int i = tid; i < q_chunks; i += 1024) {
    u32x4 x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = i + 256 * u < q_chunks ? qb[i + 256 * u] : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= x[u][0] ^ x[u][1] ^ x[u][2] ^ x[u][3];
  }
  wait_vmcnt<0>();
  __syncthreads();
  for (int i = tid * 16; i < bytes; i += 256 * 16) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(sK + i);
    const u32x4 b = *reinterpret_cast<const u32x4*>(sV + i);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3];
  }
  for (int d = 32; d >= 1; d >>= 1) acc ^= __shfl_xor(acc, d);
  if (lane == 0) sPart[wave] = acc;
  __syncthreads();
  if (tid == 0) out[blockIdx.x] = sPart[0] ^ sPart[1] ^ sPart[2] ^ sPart[3];
}

// Four independent chains of D = A.B + D per wave; ops holds, per wave of a
// workgroup, 8 fragments (A and B of each chain) of 64 lanes x 8 bf16.
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mfma_kernel(const bf16x8* __restrict__ ops, float* __restrict__ sums,
                 uint64_t* __restrict__ clocks, int iters) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const bf16x8* my = ops + wave * 8 * 64;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    a[c] = my[(2 * c) * 64 + lane];
    b[c] = my[(2 * c + 1) * 64 + lane];
  }
  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c], b[c], acc[c], 0, 0, 0);
  }
  // the last results are read before the clocks stop
  float s[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    s[c] = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[c] += acc[c][i];
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    float x = s[c];
    for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d);
    if (lane == 0) sums[((int64_t)blockIdx.x * 8 + wave) * 4 + c] = x;
  }
  if (threadIdx.x == 0) {
    clocks[2 * blockIdx.x] = t1 - t0;
    clocks[2 * blockIdx.x + 1] = r1 - r0;
  }
}

}  // namespace

int read_floor_max_keys(int hd) { return FLOOR_TENSOR_BYTES / (hd * 2); }

hipError_t launch_read_floor(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             uint32_t* out, int hd, int rows_per_group, int n_groups, int s_k,
                             int num_splits, hipStream_t stream) {
  const int tiles = (rows_per_group + 127) / 128;
  const int chunk = (s_k + num_splits - 1) / num_splits;
  const dim3 grid((unsigned)((int64_t)tiles * n_groups * num_splits));
  hipLaunchKernelGGL(read_floor_kernel, grid, dim3(256), 0, stream, q, k, v, out, hd,
                     rows_per_group, n_groups, tiles, s_k, chunk);
  return hipGetLastError();
}

hipError_t launch_mfma_ceiling(const void* ops, float* sums, uint64_t* clocks, int n_wg,
                               int iters, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_kernel, dim3((unsigned)n_wg), dim3(512), 0, stream,
                     static_cast<const bf16x8*>(ops), sums, clocks, iters);
  return hipGetLastError();
}

}  // namespace fmha
