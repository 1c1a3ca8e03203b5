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
// buffered, shared by the 4 tokens of a workgroup).  In the 32x32 output a
// lane holds one entry and 16 of the 32 heads, so the weighted ReLU sum over
// heads is in-lane plus one v_permlane32_swap.
//
// topk_kernel: one 1024-thread workgroup per token; the row's scores, mapped to
// order-preserving 32-bit keys, stay in VGPRs (32 per thread).  A 3-pass radix
// select (12, 12, 8 bits; LDS histograms, only the first pass counting every
// key) finds the top_k-th key exactly, then a pass in entry order writes every
// entry above it and the first entries equal to it: usually (every key equal
// to it kept) through a bitmap of the hits in LDS and one scan of its words'
// counts, else ranked by wave ballots and one scan of per-(chunk, wave) counts.
#include "fmha_device.h"

namespace fmha {
namespace {

using namespace dev;

// Tokens per score workgroup (one per wave).  Four, so that the two waves a
// SIMD runs come from two workgroups, whose per-tile barriers do not keep them
// in the same phase (eight: 869.7 us per bench call against 857.5; two: 964).
constexpr int IDX_WAVES = 4;
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
    constexpr int NKB = IDX_KT / 32;
    const int e0 = (tile0 + t) * IDX_KT;
    // all NKB x NHB accumulators at once: independent MFMA chains, each K
    // fragment read once for every head block
    f32x16 s[NKB][NHB];
#pragma unroll
    for (int cs = 0; cs < NCS; ++cs) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(buf + k_lane + kb * 32 * KS + cs * 32);
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
          const f32x16 zero = {};
          s[kb][hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[hb][cs], b,
                                                              cs == 0 ? zero : s[kb][hb], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      float a[4] = {0.f, 0.f, 0.f, 0.f};  // four partial sums: short dependency chains
      // ReLU as one integer max of the bit pattern with 0 (a set sign bit is a
      // negative int: -x and -0 become +0, the rest is kept); fmaxf compiled
      // to two v_max_f32 per value, the first quieting a signalling NaN that
      // an MFMA result cannot be
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float relu = __int_as_float(max(__float_as_int(s[kb][hb][r]), 0));
          a[r & 3] = fmaf(wr[hb][r], relu, a[r & 3]);
        }
      const float acc = pair_sum((a[0] + a[1]) + (a[2] + a[3]));
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
constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / 64;
constexpr int SEL_MAX_P = 32768;                 // a row's keys fit in VGPRs
constexpr int SEL_J = SEL_MAX_P / SEL_THREADS;   // keys per thread
constexpr int SEL_BINS = 4096;                   // 12-bit digits (the last pass: 8)
constexpr int SEL_CAND = 2048;  // boundary-digit keys kept in LDS for passes 2 and 3

// Order-preserving map of a float score to a 32-bit key (-0 and +0 equal).
__device__ __forceinline__ uint32_t order_key(float f) {
  f += 0.f;
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP: shifts within
// each 16-lane row, then row broadcasts of lane 15 and lane 31 (GFX9 DPP).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  int x = (int)v;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false); // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false); // row_bcast:31 -> rows 2, 3
  return (uint32_t)x;
}

// Sums of wtot[0 .. nw) over the waves before this one and over all of them,
// by one more wave scan (lane l holds wtot[l]) and two readlanes.
__device__ __forceinline__ void wave_totals(const uint32_t* wtot, int nw, uint32_t& before,
                                            uint32_t& total) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t incl = wave_incl_scan(lane < nw ? wtot[lane] : 0u);
  total = (uint32_t)__builtin_amdgcn_readlane((int)incl, nw - 1);
  before = wave > 0 ? (uint32_t)__builtin_amdgcn_readlane((int)incl, wave - 1) : 0u;
}

// One radix step: `hist` holds the digit counts of the keys that share the
// prefix found so far; find the digit of the krem-th largest of them (the
// highest digit b with count(> b) < krem <= count(>= b)) and record the new
// prefix, the rank left in it and the digit's count in s[0], s[1], s[2].  NB digits, NB / SEL_THREADS per thread
// (or one digit for the first NB threads).  Starts and ends with a barrier's
// worth of ordering: every thread must call it.
template <int NB>
__device__ __forceinline__ void radix_step(const int* hist, uint32_t* wtot, uint32_t* s,
                                           uint32_t prefix, int shift, int krem) {
  constexpr int BPT = NB >= SEL_THREADS ? NB / SEL_THREADS : 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool owner = tid * BPT < NB;
  int c[BPT];
  uint32_t mine = 0;
#pragma unroll
  for (int b = 0; b < BPT; ++b) {
    c[b] = owner ? hist[tid * BPT + b] : 0;
    mine += c[b];
  }
  const uint32_t incl = wave_incl_scan(mine);
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  uint32_t before, total;
  wave_totals(wtot, SEL_WAVES, before, total);
  // keys in digits above this thread's: everything after it in digit order
  int cum = (int)(total - (before + incl));
#pragma unroll
  for (int b = BPT - 1; b >= 0; --b) {
    if (owner && cum < krem && cum + c[b] >= krem) {
      s[0] = prefix | ((uint32_t)(tid * BPT + b) << shift);
      s[1] = (uint32_t)(krem - cum);
      s[2] = (uint32_t)c[b];
    }
    cum += c[b];
  }
  __syncthreads();
}

// Keeps the compiler from reusing one loop's comparisons in a later loop
// (64 ballot masks would spill); recomputing them costs one VALU each.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

__global__ __launch_bounds__(SEL_THREADS) void topk_kernel(const float* __restrict__ scores,
                                                           int32_t* __restrict__ idx, int P,
                                                           int top_k) {
  __shared__ int histA[SEL_BINS];
  __shared__ int histB[SEL_BINS];
  __shared__ uint32_t cand[SEL_CAND];
  __shared__ uint32_t cnt[SEL_J * SEL_WAVES];  // per (chunk, wave) counts, then their prefix
  __shared__ uint32_t wtot[SEL_WAVES];
  __shared__ uint32_t s_sel[3];                // prefix, rank left in it, its digit's count
  __shared__ int s_ncand;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const float* src = scores + row * P;
  int32_t* dst = idx + row * top_k;
  const int n = min(top_k, P);
  for (int i = n + tid; i < top_k; i += SEL_THREADS) dst[i] = -1;
  if (n <= 0) return;

  // The histograms are cleared before the row is loaded, so that pass 1 can
  // count each key as soon as its own load has landed (the loads return in
  // order) while the later loads are still in flight.
  const int pad = SEL_MAX_P - P;
#pragma unroll
  for (int b = 0; b < SEL_BINS / SEL_THREADS; ++b) {
    histA[b * SEL_THREADS + tid] = 0;
    histB[b * SEL_THREADS + tid] = 0;
  }
  if (tid == 0) s_ncand = 0;
  __syncthreads();

  // key j of this thread is entry j * SEL_THREADS + tid (coalesced loads).
  // Buffer loads (past the row's end they read zero) with one shared 32-bit
  // offset: no predication and no per-load address, so all SEL_J loads are in
  // flight together.
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, P * 4, BUF_FLAGS);
  uint32_t u[SEL_J];
#pragma unroll
  for (int j = 0; j < SEL_J; ++j)
    u[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, tid * 4, j * SEL_THREADS * 4, 0);
  // Entries past the row's end get key 0, the smallest key.  Rather than test
  // validity per key in every pass, their count (pad) is taken back out of
  // digit 0 in each pass whose prefix they share; in entry order they come
  // after every real entry, so the compaction never selects them.
  const int jn = (P - tid + SEL_THREADS - 1) / SEL_THREADS;  // this thread's real keys
  const int jfull = P / SEL_THREADS;                         // chunks real for every thread

  // pass 1: bits 31..20 of every key, each counted as it arrives
  if (tid == 0) atomicAdd(&histA[0], -pad);
#pragma unroll
  for (int j = 0; j < SEL_J; ++j) {
    uint32_t key = order_key(__uint_as_float(u[j]));
    if (j >= jfull && j >= jn) key = 0u;
    u[j] = key;
    atomicAdd(&histA[key >> 20], 1);
  }
  __syncthreads();
  radix_step<SEL_BINS>(histA, wtot, s_sel, 0u, 20, n);
  uint32_t prefix = s_sel[0];
  int krem = (int)s_sel[1];
  const int c1 = (int)s_sel[2];  // keys in the boundary digit
  if (tid < 256) histA[tid] = 0;  // pass 1's counts were all read before the step's last barrier

  // Passes 2 and 3 only look at the boundary digit's keys: gathered into LDS
  // when few (and not sharing digit 0 with the padding), else re-scanned in
  // VGPRs.
  const bool use_cand = c1 <= SEL_CAND && (prefix >> 20) != 0;
  if (use_cand) {
#pragma unroll
    for (int j = 0; j < SEL_J; ++j)
      if ((u[j] ^ prefix) < (1u << 20)) cand[atomicAdd(&s_ncand, 1)] = u[j];
    __syncthreads();
    for (int k = tid; k < c1; k += SEL_THREADS)
      atomicAdd(&histB[(cand[k] >> 8) & (SEL_BINS - 1)], 1);
  } else {
    if (tid == 0 && (prefix >> 20) == 0) atomicAdd(&histB[0], -pad);
#pragma unroll
    for (int j = 0; j < SEL_J; ++j)
      if ((u[j] ^ prefix) < (1u << 20)) atomicAdd(&histB[(u[j] >> 8) & (SEL_BINS - 1)], 1);
  }
  __syncthreads();
  radix_step<SEL_BINS>(histB, wtot, s_sel, prefix, 8, krem);
  prefix = s_sel[0];
  krem = (int)s_sel[1];

  // pass 3: bits 7..0
  if (use_cand) {
    for (int k = tid; k < c1; k += SEL_THREADS) {
      const uint32_t v = cand[k];
      if ((v ^ prefix) < 256u) atomicAdd(&histA[v & 255], 1);
    }
  } else {
    if (tid == 0 && (prefix >> 8) == 0) atomicAdd(&histA[0], -pad);
#pragma unroll
    for (int j = 0; j < SEL_J; ++j)
      if ((u[j] ^ prefix) < 256u) atomicAdd(&histA[u[j] & 255], 1);
  }
  __syncthreads();
  radix_step<256>(histA, wtot, s_sel, prefix, 0, krem);
  const uint32_t T = s_sel[0];        // the n-th largest key
  const int take_eq = (int)s_sel[1];  // how many keys equal to T are kept (the first ones)
  const int n_eq = (int)s_sel[2];     // how many keys equal T

  // Ordered compaction: entries above T and the first take_eq entries equal
  // to T, in entry order.  Per (chunk, wave) counts, one exclusive scan of
  // them in entry order, then in-wave ranks from the ballots.  Usually every
  // key equal to T is kept (T > 0 then also excludes the padding): one mask,
  // u >= T.  Otherwise the ranks of the keys above T and equal to T are kept
  // apart (packed gt | eq << 16; each count fits 16 bits, so the packed sums
  // do not carry).
  const bool all_eq = take_eq == n_eq && T != 0u;
  const __amdgpu_buffer_rsrc_t rd =
      __builtin_amdgcn_make_buffer_rsrc((void*)dst, (short)0, n * 4, BUF_FLAGS);
  if (all_eq) {
    // The usual case, by a bitmap of the hits in entry order (in pass 2's
    // histogram, free by now): entries j*SEL_THREADS + 64*wave + lane of
    // chunk j are the bits of words 32j + 2*wave (+1), one 8-byte write per
    // (chunk, wave).  Thread t then owns word t (entries 32t .. 32t+31): one
    // block scan of the words' counts, and its few hits go out in order.
    // Measured 6% faster per call than the ballot ranks below.
    static_assert(SEL_MAX_P == 32 * SEL_THREADS && SEL_BINS >= SEL_MAX_P / 32, "one word a thread");
    uint32_t* bits = reinterpret_cast<uint32_t*>(histB);
#pragma unroll
    for (int j = 0; j < SEL_J; ++j) {
      const uint64_t m = __ballot(u[j] >= T);
      if (lane == 0)
        *reinterpret_cast<uint2*>(bits + j * (SEL_THREADS / 32) + 2 * wave) =
            make_uint2((uint32_t)m, (uint32_t)(m >> 32));
    }
    __syncthreads();
    uint32_t word = bits[tid];
    const uint32_t cw = (uint32_t)__popc(word);
    const uint32_t incl = wave_incl_scan(cw);
    if (lane == 63) wtot[wave] = incl;
    __syncthreads();
    uint32_t before, total;
    wave_totals(wtot, SEL_WAVES, before, total);
    uint32_t pos = before + incl - cw;
    while (word) {
      const int b = __builtin_ctz(word);
      word &= word - 1;
      __builtin_amdgcn_raw_buffer_store_b32((uint32_t)(tid * 32 + b), rd, (int)(pos * 4), 0, 0);
      ++pos;
    }
    return;
  }
  uint32_t my_cnt = 0;  // lane j: this wave's count in chunk j
#pragma unroll
  for (int j = 0; j < SEL_J; ++j) {
    uint32_t c;
    if (all_eq) {
      c = (uint32_t)__popcll(__ballot(u[j] >= T));
    } else {
      c = (uint32_t)__popcll(__ballot(u[j] > T)) |
          ((uint32_t)__popcll(__ballot(u[j] == T)) << 16);
    }
    asm("v_writelane_b32 %0, %1, m0" : "+v"(my_cnt) : "s"(c), "{m0}"(j));
  }
  if (lane < SEL_J) cnt[lane * SEL_WAVES + wave] = my_cnt;
  __syncthreads();
  constexpr int NC = SEL_J * SEL_WAVES;
  static_assert(NC <= SEL_THREADS && SEL_J <= 64, "one count per thread");
  uint32_t v = 0, incl = 0;
  if (tid < NC) {
    v = cnt[tid];
    incl = wave_incl_scan(v);
    if (lane == 63) wtot[wave] = incl;
  }
  __syncthreads();
  if (tid < NC) {
    uint32_t before, total;
    wave_totals(wtot, NC / 64, before, total);
    cnt[tid] = before + incl - v;  // exclusive prefix; each thread rewrites only its own entry
  }
  __syncthreads();
  const uint32_t basev = lane < SEL_J ? cnt[lane * SEL_WAVES + wave] : 0u;  // lane j: chunk j's base
  const uint32_t T2 = opaque(T);
#pragma unroll
  for (int j = 0; j < SEL_J; ++j) {
    const uint32_t base = (uint32_t)__builtin_amdgcn_readlane((int)basev, j);
    const uint32_t id = (uint32_t)(j * SEL_THREADS + tid);
    if (all_eq) {
      const bool hit = u[j] >= T2;
      const uint64_t m = __ballot(hit);
      const uint32_t pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, base));
      if (hit) __builtin_amdgcn_raw_buffer_store_b32(id, rd, (int)(pos * 4), 0, 0);
    } else {
      const bool gt = u[j] > T2, eq = u[j] == T2;
      const uint64_t mg = __ballot(gt), me = __ballot(eq);
      const int gt_before = (int)__builtin_amdgcn_mbcnt_hi(
          (uint32_t)(mg >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mg, base & 0xffffu));
      const int eq_before = (int)__builtin_amdgcn_mbcnt_hi(
          (uint32_t)(me >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)me, base >> 16));
      if (gt || (eq && eq_before < take_eq))
        __builtin_amdgcn_raw_buffer_store_b32(id, rd, (gt_before + min(eq_before, take_eq)) * 4,
                                              0, 0);
    }
  }
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
