// Top-k indexer for gfx950: the gather lists (kv_idx) the sparse attention
// reads.
//
// The dsv4/kernels/cuda commit log (indexer_score_topk) forms index scores per
// index head with per-head weights and keeps the 1024 best pool entries per
// token, checked by exact match against torch.topk; it does not print the
// score formula.  Reading taken (the DeepSeek sparse-attention indexer form,
// one index key per pool entry shared by the heads):
//   score[t, s] = sum_h w[t, h] * max(0, q[t, h, :] . k[s, :])
// and the selection keeps the top_k largest scores (ties towards the smaller
// entry id), listed in ascending entry-id order, -1 padding when P < top_k.
//
// score_kernel: S = Q_t . K^T with v_mfma_f32_32x32x16_bf16, the A operand
// being 32 index heads of one token (Q in VGPRs for the whole kernel) and the
// B operand 32 pool entries (K tiles moved global -> LDS by LDS-DMA, double
// buffered, shared by the 8 tokens of a workgroup).  In the 32x32 output a
// lane holds one entry and 16 of the 32 heads, so the weighted ReLU sum over
// heads is in-lane plus one v_permlane32_swap.
//
// topk_kernel: one workgroup per token; the row's scores, mapped to
// order-preserving 32-bit keys, sit in LDS; a 4-pass radix select (8 bits per
// pass, LDS histograms) finds the top_k-th key exactly, then a pass in entry
// order writes every entry above it and the first entries equal to it, with
// wave ballots for the prefix counts.
#include "fmha_device.h"

namespace fmha {
namespace {

using namespace dev;

constexpr int IDX_WAVES = 8;  // tokens per score workgroup (one per wave)
constexpr int IDX_KT = 64;    // pool entries per K tile
constexpr uint32_t IDX_OOB = 0x80000000u;

template <int C>
struct IdxLds {
  static constexpr int ROW = C * 2;
  static constexpr int STRIDE = ROW + 16;  // conflict-free ds_read_b128 of 16 rows
  static constexpr int NI = (IDX_KT * STRIDE + 1023) / 1024;  // DMA instructions per tile
};

// DMA of the K tile that starts at pool entry e0 into `buf` (entries past P
// read as zeros): instruction j of wave `wave` fills LDS bytes
// [1024 (wave + 8 j), +1024); off[j] is the lane's byte offset in the tile.
template <int C, int J, int NI>
__device__ __forceinline__ void issue_tile(const uint16_t* k, int P, int e0, char* buf, int wave,
                                           const uint32_t* off) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(k + (int64_t)e0 * C), (short)0, (P - e0) * (C * 2), BUF_FLAGS);
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int inst = wave + IDX_WAVES * j;
    if (inst < NI)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(buf + inst * 1024), 16, off[j], 0, 0, 0);
  }
}

template <int C, int H>
__global__ __launch_bounds__(IDX_WAVES * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void score_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                  const float* __restrict__ wt, float* __restrict__ scores, int tokens, int P,
                  int tiles_per_wg) {
  constexpr int NHB = H / 32;   // 32-head row blocks
  constexpr int NCS = C / 16;   // contraction steps
  constexpr int ROW = IdxLds<C>::ROW;
  constexpr int KS = IdxLds<C>::STRIDE;
  constexpr int NI = IdxLds<C>::NI;
  constexpr int J = (NI + IDX_WAVES - 1) / IDX_WAVES;
  __shared__ __attribute__((aligned(1024))) char sK0[NI * 1024], sK1[NI * 1024];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hlf = lane >> 5;
  const int token = blockIdx.x * IDX_WAVES + wave;
  const bool live = token < tokens;
  const int tile0 = blockIdx.y * tiles_per_wg;
  const int n_tiles = max(0, min(tiles_per_wg, (P + IDX_KT - 1) / IDX_KT - tile0));

  // Q rows (heads) of this wave's token as MFMA A fragments; head weights in
  // the output layout (register r of block hb holds head 32 hb + 8 (r/4) +
  // 4 hlf + r%4).
  bf16x8 qf[NHB][NCS];
  float wr[NHB][16];
  const int tq = live ? token : 0;
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const uint16_t* qrow = q + ((int64_t)tq * H + hb * 32 + l32) * C + 8 * hlf;
#pragma unroll
    for (int cs = 0; cs < NCS; ++cs)
      qf[hb][cs] = *reinterpret_cast<const bf16x8*>(qrow + 16 * cs);
#pragma unroll
    for (int r = 0; r < 16; ++r) wr[hb][r] = wt[(int64_t)tq * H + hb * 32 + acc_row(r, hlf)];
  }

  // DMA geometry: instruction j of this wave fills LDS bytes
  // [1024 (wave + 8 j), +1024) of a tile buffer; lane -> (row, column byte).
  uint32_t off[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int pos = (wave + IDX_WAVES * j) * 1024 + lane * 16;
    const int r = pos / KS, cc = pos % KS;
    off[j] = (cc < ROW && r < IDX_KT) ? (uint32_t)(r * ROW + cc) : IDX_OOB;
  }
  auto issue = [&](int t, char* buf) __attribute__((always_inline)) {
    issue_tile<C, J, NI>(k, P, (tile0 + t) * IDX_KT, buf, wave, off);
  };

  const int k_lane = l32 * KS + 16 * hlf;
  auto compute = [&](int t, const char* buf) __attribute__((always_inline)) {
    const int e0 = (tile0 + t) * IDX_KT;
#pragma unroll
    for (int kb = 0; kb < IDX_KT / 32; ++kb) {
      float acc = 0.f;
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        f32x16 s = {};
#pragma unroll
        for (int cs = 0; cs < NCS; ++cs) {
          const bf16x8 b = *reinterpret_cast<const bf16x8*>(buf + k_lane + kb * 32 * KS + cs * 32);
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[hb][cs], b, s, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) acc = fmaf(wr[hb][r], fmaxf(s[r], 0.f), acc);
      }
      acc = pair_sum(acc);
      const int e = e0 + kb * 32 + l32;
      if (live && hlf == 0 && e < P) scores[(int64_t)token * P + e] = acc;
    }
  };

  if (n_tiles > 0) {
    issue(0, sK0);
    __syncthreads();
  }
  for (int t = 0; t < n_tiles; t += 2) {
    if (t + 1 < n_tiles) issue(t + 1, sK1);
    compute(t, sK0);
    __syncthreads();  // tile t+1 landed; sK0 free
    if (t + 1 < n_tiles) {
      if (t + 2 < n_tiles) issue(t + 2, sK0);
      compute(t + 1, sK1);
      __syncthreads();
    }
  }
}

// ------------------------------------------------------------- selection
constexpr int SEL_THREADS = 256;
constexpr int SEL_MAX_P = 32768;  // a row's keys fit in LDS (128 KiB)

// Order-preserving map of a float to uint32 (-0 taken as +0).
__device__ __forceinline__ uint32_t order_key(float f) {
  f += 0.f;
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Exclusive prefix count of `flag` over the workgroup's threads in thread
// order, and the workgroup total (every thread calls it; uses wsum[4]).
__device__ __forceinline__ int block_prefix(bool flag, int* wsum, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t m = __ballot(flag);
  const int in_wave = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
  if (lane == 0) wsum[wave] = __popcll(m);
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < SEL_THREADS / 64; ++w) {
    const int c = wsum[w];
    before += w < wave ? c : 0;
    total += c;
  }
  __syncthreads();  // wsum reused by the next call
  return before + in_wave;
}

__global__ __launch_bounds__(SEL_THREADS) void topk_kernel(const float* __restrict__ scores,
                                                           int32_t* __restrict__ idx, int P,
                                                           int top_k) {
  __shared__ uint32_t sKey[SEL_MAX_P];
  __shared__ int hist[256];
  __shared__ int wsum[SEL_THREADS / 64];
  __shared__ uint32_t s_prefix;
  __shared__ int s_krem;

  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const float* src = scores + row * P;
  int32_t* dst = idx + row * top_k;
  const int n = min(top_k, P);
  if (n <= 0) {
    for (int i = tid; i < top_k; i += SEL_THREADS) dst[i] = -1;
    return;
  }

  for (int i = tid; i < P; i += SEL_THREADS) sKey[i] = order_key(src[i]);
  if (tid == 0) {
    s_prefix = 0;
    s_krem = n;
  }
  __syncthreads();

  // radix select of the n-th largest key, most significant byte first
  uint32_t mask = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += SEL_THREADS) hist[i] = 0;
    __syncthreads();
    const uint32_t prefix = s_prefix;
    for (int i = tid; i < P; i += SEL_THREADS) {
      const uint32_t u = sKey[i];
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255], 1);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l owns bins 4l .. 4l+3; suffix sums from the top bin down
      const int lane = tid;
      const int c0 = hist[4 * lane], c1 = hist[4 * lane + 1], c2 = hist[4 * lane + 2],
                c3 = hist[4 * lane + 3];
      const int mine = c0 + c1 + c2 + c3;
      int suf = mine;  // inclusive suffix sum over lanes lane .. 63
      for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_down(suf, d);
        if (lane + d < 64) suf += o;
      }
      const int above = suf - mine;  // keys in bins owned by higher lanes
      const int krem = s_krem;
      // the bin holding the krem-th largest: the highest bin b with
      // count(bins > b) < krem <= count(bins >= b)
      int found = -1, newk = 0;
      int cum = above;
      const int c[4] = {c0, c1, c2, c3};
#pragma unroll
      for (int b = 3; b >= 0; --b) {
        if (found < 0 && cum < krem && cum + c[b] >= krem) {
          found = 4 * lane + b;
          newk = krem - cum;
        }
        cum += c[b];
      }
      const uint64_t who = __ballot(found >= 0);
      const int src_lane = 63 - __builtin_clzll(who);
      const int bin = __shfl(found, src_lane);
      const int k2 = __shfl(newk, src_lane);
      if (lane == 0) {
        s_prefix = prefix | ((uint32_t)bin << shift);
        s_krem = k2;
      }
    }
    __syncthreads();
    mask |= 255u << shift;
  }
  const uint32_t T = s_prefix;   // the n-th largest key
  const int take_eq = s_krem;    // how many keys equal to T are kept
  __syncthreads();

  // entries above T, and the first take_eq entries equal to T, in entry order
  int eq_run = 0, sel_run = 0;
  for (int base = 0; base < P; base += SEL_THREADS) {
    const int i = base + tid;
    const uint32_t u = i < P ? sKey[i] : 0u;
    const bool gt = i < P && u > T;
    const bool eq = i < P && u == T;
    int eq_tot, sel_tot;
    const int eq_before = eq_run + block_prefix(eq, wsum, eq_tot);
    const bool sel = gt || (eq && eq_before < take_eq);
    const int pos = sel_run + block_prefix(sel, wsum, sel_tot);
    if (sel) dst[pos] = i;
    eq_run += eq_tot;
    sel_run += sel_tot;
  }
  for (int i = n + tid; i < top_k; i += SEL_THREADS) dst[i] = -1;
}

template <int C, int H>
hipError_t launch_scores_t(const uint16_t* q, const uint16_t* k, const float* w, float* scores,
                           int tokens, int P, hipStream_t stream) {
  const int tok_groups = (tokens + IDX_WAVES - 1) / IDX_WAVES;
  const int total_tiles = (P + IDX_KT - 1) / IDX_KT;
  // enough workgroups to fill the chip: split the pool when tokens are few
  int chunks = (1024 + tok_groups - 1) / tok_groups;
  chunks = max(1, min(chunks, total_tiles));
  const int tiles_per_wg = (total_tiles + chunks - 1) / chunks;
  chunks = (total_tiles + tiles_per_wg - 1) / tiles_per_wg;
  hipLaunchKernelGGL((score_kernel<C, H>), dim3(tok_groups, chunks), dim3(IDX_WAVES * 64), 0,
                     stream, q, k, w, scores, tokens, P, tiles_per_wg);
  return hipGetLastError();
}

}  // namespace

int topk_max_pool() { return SEL_MAX_P; }

hipError_t launch_index_scores(const uint16_t* q, const uint16_t* k, const float* w,
                               float* scores, int tokens, int H, int C, int P,
                               hipStream_t stream) {
  if (C == 128 && H == 64) return launch_scores_t<128, 64>(q, k, w, scores, tokens, P, stream);
  if (C == 128 && H == 32) return launch_scores_t<128, 32>(q, k, w, scores, tokens, P, stream);
  if (C == 64 && H == 64) return launch_scores_t<64, 64>(q, k, w, scores, tokens, P, stream);
  if (C == 64 && H == 32) return launch_scores_t<64, 32>(q, k, w, scores, tokens, P, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_topk(const float* scores, int32_t* idx, int rows, int P, int top_k,
                       hipStream_t stream) {
  hipLaunchKernelGGL(topk_kernel, dim3(rows), dim3(SEL_THREADS), 0, stream, scores, idx, P,
                     top_k);
  return hipGetLastError();
}

}  // namespace fmha
