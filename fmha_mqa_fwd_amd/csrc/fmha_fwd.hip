// Multi-query attention forward for gfx950 (MI355X, CDNA4).
//
// What is computed follows the dev-log pages of the DeepSeek-V4 NVFP4 kernel
// project:
//   * QK^T -> softmax -> PV -> output, the QK product unscaled and the
//     1/sqrt(hd) factor applied in the softmax (page "CURRENT ISSUE: UMMA FMHA —
//     Full Pipeline + Production", "What's working" and "Key lessons from this
//     session");
//   * multi-query: every query head of a batch/token reads one shared K/V head
//     (page "May 24, 2026 — Session Start Plan", 3 "Start D2: Multi-Query Grid");
//   * keys processed tile by tile with the running O rescaled whenever the row
//     maximum grows (same page, 2 "Test O Rescale at s_k > 128");
//   * O and the row log-sum-exp as outputs (same page, "D1 Status Summary");
//   * optional row gather of the s_k = top_k selected keys from a KV pool (same
//     page "Key Numbers"; dsv4/kernels/cuda commit log, KV row gather).
//
// How it is mapped onto CDNA4 (our design, not the pages' Blackwell one):
//   * Head-packed M: the rows of a group (all (t, h) of a batch, or all heads of
//     a token) share K/V, so a workgroup takes WAVES*QW consecutive rows and
//     every K/V tile staged in LDS serves all of them.
//   * S^T = K . Q^T with v_mfma_f32_32x32x16_bf16: K (A operand) comes from LDS,
//     Q^T (B operand) stays in VGPRs for the whole kernel.  In the 32x32
//     accumulator layout lane l holds query column l%32 and 16 of the 32 keys,
//     so a row's max/sum is an in-lane reduction plus one exchange with lane
//     l^32, and the per-row rescale factor is a per-lane scalar.
//   * O^T = V^T . P^T: the S^T accumulators, rounded to bf16, are already the B
//     operand of the PV MFMA (no LDS round trip for P).  V^T is written to LDS
//     transposed while staging, in the key order that the accumulator layout
//     implies, so the A operand is one 16-byte LDS read.
//   * Online softmax in base 2: x*scale*log2(e) folded into one FMA, exp2 on
//     the hardware transcendental unit, fp32 row max/sum.
//   * LDS tiles use an XOR swizzle of 16-byte chunks so the MFMA operand reads
//     and the staging writes do not collide on banks.
#include <math.h>

#include "fmha_internal.h"

namespace fmha {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int WAVES = 4;
constexpr int THREADS = WAVES * 64;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// Physical 16-byte chunk for logical chunk c of LDS row `row`, for rows of CPR
// chunks.  16+ chunks per row: XOR the low 4 bits with row ^ row>>3 (rows that
// an MFMA operand read touches together, 32 consecutive rows, and the rows a
// transposed staging write touches, rows 8 apart, both land on distinct
// chunks).  8 chunks per row (128-byte rows, two per 256 bytes): XOR with
// (row & 7) ^ (row>>3 & 1).
template <int CPR>
__device__ __forceinline__ int swz(int row) {
  static_assert(CPR >= 8, "LDS rows must hold at least 8 chunks");
  if constexpr (CPR >= 16) {
    return (row ^ (row >> 3)) & 15;
  } else {
    return (row & 7) ^ ((row >> 3) & 1);
  }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  __bf16 x = (__bf16)a;  // round to nearest even (v_cvt_pk_bf16_f32)
  __bf16 y = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) |
         ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

__device__ __forceinline__ bf16x8 pack_bf16x8(const float* s) {
  u32x4 w;
  w[0] = pack_bf16x2(s[0], s[1]);
  w[1] = pack_bf16x2(s[2], s[3]);
  w[2] = pack_bf16x2(s[4], s[5]);
  w[3] = pack_bf16x2(s[6], s[7]);
  return __builtin_bit_cast(bf16x8, w);
}

// Key (within a 32-key block) held by accumulator register r of a lane in
// half `hlf` of the wave, for the 32x32 MFMA output layout (rows grouped in
// fours: register r covers row 8*(r/4) + 4*hlf + r%4, column lane%32).
__device__ __forceinline__ int acc_row(int r, int hlf) {
  return 8 * (r >> 2) + 4 * hlf + (r & 3);
}

template <int HD, int QW, int KT, bool GATHER>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fwd_kernel(FwdParams p) {
  constexpr int NQB = QW / 32;   // 32-query MFMA column blocks per wave
  constexpr int NDS = HD / 16;   // 16-wide contraction steps of QK^T
  constexpr int NKB = KT / 32;   // 32-key row blocks of S^T per tile
  constexpr int NKS = KT / 16;   // 16-key contraction steps of PV per tile
  constexpr int NDB = HD / 32;   // 32-wide d blocks of O^T
  constexpr int K_CPR = HD / 8;  // 16-byte chunks per K row in LDS
  constexpr int V_CPR = KT / 8;  // 16-byte chunks per V^T row in LDS
  constexpr int M_WG = WAVES * QW;
  static_assert(QW % 32 == 0 && KT % 32 == 0 && HD % 32 == 0, "tile shape");

  __shared__ __attribute__((aligned(16))) uint16_t sK[KT * HD];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[HD * KT];
  __shared__ int sIdx[KT];  // pool row per tile key, -1 = masked

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hlf = lane >> 5;

  int bid = blockIdx.x;
  const int tile = bid % p.tiles_per_group;
  bid /= p.tiles_per_group;
  const int group = bid % p.n_groups;
  const int split = bid / p.n_groups;

  const int key_lo = split * p.chunk;
  const int key_hi = min(key_lo + p.chunk, p.s_k);
  const int row0 = tile * M_WG + wave * QW;  // first row of this wave in its group
  const int64_t grow0 = (int64_t)group * p.rows_per_group;

  // Q^T fragments (B operand of S^T = K.Q^T): lane (hlf, l32) of column block
  // qb holds q[row l32][16*ds + 8*hlf .. +7] for every contraction step ds.
  bf16x8 qf[NQB][NDS];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int r = row0 + qb * 32 + l32;
    const bool ok = r < p.rows_per_group;
    const uint16_t* qrow = p.q + (grow0 + (ok ? r : 0)) * HD + 8 * hlf;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (ok) w = *reinterpret_cast<const u32x4*>(qrow + 16 * ds);
      qf[qb][ds] = __builtin_bit_cast(bf16x8, w);
    }
  }

  f32x16 o[NDB][NQB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][qb][i] = 0.f;
  float m[NQB], l[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    m[qb] = neg_inf();
    l[qb] = 0.f;
  }

  const float c = p.scale_log2;

  for (int t0 = key_lo; t0 < key_hi; t0 += KT) {
    __syncthreads();  // every wave is done with the previous tile's LDS

    // ---- which pool row (gather) or key (dense) each tile row holds
    int masked = 0;
    if constexpr (GATHER) {
      for (int j = tid; j < KT; j += THREADS) {
        const int key = t0 + j;
        int idx = -1;
        if (key < key_hi) {
          idx = p.kv_idx[(int64_t)group * p.s_k + key];
          if (idx < 0 || idx >= p.pool_rows) idx = -1;
        }
        sIdx[j] = idx;
        masked |= (idx < 0);
      }
      masked = __syncthreads_or(masked);
    } else {
      masked = (t0 + KT > key_hi);
      for (int j = tid; j < KT; j += THREADS) sIdx[j] = (t0 + j < key_hi) ? 0 : -1;
      __syncthreads();
    }

    // ---- K tile: [KT rows][HD], row j = key t0+j, 16-byte chunks swizzled
    for (int u = tid; u < KT * K_CPR; u += THREADS) {
      const int row = u / K_CPR;
      const int ch = u % K_CPR;
      u32x4 w = {0u, 0u, 0u, 0u};
      const int idx = sIdx[row];
      if (idx >= 0) {
        const uint16_t* src = GATHER ? p.k + (int64_t)idx * HD
                                     : p.k + ((int64_t)group * p.s_k + t0 + row) * HD;
        w = *reinterpret_cast<const u32x4*>(src + 8 * ch);
      }
      *reinterpret_cast<u32x4*>(sK + row * HD + 8 * (ch ^ swz<K_CPR>(row))) = w;
    }

    // ---- V^T tile: [HD rows][KT keys].  Chunk (2*ks + hh) of row d holds the
    // keys 16*ks + 8*(e/4) + 4*hh + e%4, e = 0..7: exactly the keys that lanes
    // of half hh hold, in register order, in S^T's accumulators.
    for (int u = tid; u < (HD / 8) * NKS * 2; u += THREADS) {
      const int dc = u % (HD / 8);
      const int rest = u / (HD / 8);
      const int hh = rest & 1;
      const int ks = rest >> 1;
      u32x4 in[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = 16 * ks + 8 * (e >> 2) + 4 * hh + (e & 3);
        const int idx = sIdx[j];
        in[e] = u32x4{0u, 0u, 0u, 0u};
        if (idx >= 0) {
          const uint16_t* src = GATHER ? p.v + (int64_t)idx * HD
                                       : p.v + ((int64_t)group * p.s_k + t0 + j) * HD;
          in[e] = *reinterpret_cast<const u32x4*>(src + 8 * dc);
        }
      }
      const int cv = 2 * ks + hh;
#pragma unroll
      for (int di = 0; di < 8; ++di) {
        u32x4 w;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const uint32_t lo = in[2 * a][di >> 1];
          const uint32_t hi = in[2 * a + 1][di >> 1];
          w[a] = (di & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
        }
        const int d = 8 * dc + di;
        *reinterpret_cast<u32x4*>(sVt + d * KT + 8 * (cv ^ swz<V_CPR>(d))) = w;
      }
    }
    __syncthreads();

    // ---- S^T = K . Q^T  (unscaled dot products, fp32)
    f32x16 s[NKB][NQB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][qb][i] = 0.f;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int row = 32 * kb + l32;
        const int ch = 2 * ds + hlf;
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(sK + row * HD + 8 * (ch ^ swz<K_CPR>(row)));
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
          s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][ds], s[kb][qb], 0, 0, 0);
      }
    }
    if (masked) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (sIdx[32 * kb + acc_row(r, hlf)] < 0) {
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) s[kb][qb][r] = neg_inf();
          }
        }
    }

    // ---- online softmax (base 2) and O rescale
    bf16x8 pf[NQB][NKS];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      float mx = neg_inf();
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m[qb], mx * c);
      const float m_use = (m_new == neg_inf()) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m[qb] - m_use);
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        float pv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          pv[r] = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][r], c, -m_use));
          ls += pv[r];
        }
        pf[qb][2 * kb] = pack_bf16x8(pv);
        pf[qb][2 * kb + 1] = pack_bf16x8(pv + 8);
      }
      l[qb] = l[qb] * alpha + ls;
      m[qb] = m_new;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][qb][i] *= alpha;
    }

    // ---- O^T += V^T . P^T
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int d = 32 * db + l32;
        const int ch = 2 * ks + hlf;
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(sVt + d * KT + 8 * (ch ^ swz<V_CPR>(d)));
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
          o[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[qb][ks], o[db][qb], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: O / l, lse = (m + log2 l) * ln 2
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const float lt = l[qb] + __shfl_xor(l[qb], 32);
    const bool empty = (m[qb] == neg_inf());
    const float inv = empty ? 0.f : 1.f / lt;
    const float lse_v = empty ? neg_inf() : (m[qb] + log2f(lt)) * LN2;
    const int r = row0 + qb * 32 + l32;
    if (r >= p.rows_per_group) continue;
    const int64_t row = grow0 + r;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d = 32 * db + 8 * rg + 4 * hlf;
        f32x4 val;
#pragma unroll
        for (int i = 0; i < 4; ++i) val[i] = o[db][qb][4 * rg + i] * inv;
        if (p.out_mode == OUT_BF16) {
          u32x2 w = {pack_bf16x2(val[0], val[1]), pack_bf16x2(val[2], val[3])};
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.out) + row * HD + d) = w;
        } else {
          const int64_t base = (p.out_mode == OUT_PARTIAL) ? (int64_t)split * p.total_rows : 0;
          *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + (base + row) * HD + d) = val;
        }
      }
    }
    if (hlf == 0) {
      const int64_t base = (p.out_mode == OUT_PARTIAL) ? (int64_t)split * p.total_rows : 0;
      p.lse[base + row] = lse_v;
    }
  }
}

struct Shape {
  int qw, kt;
};

// 64 rows per wave (256 per workgroup) halves the LDS operand traffic per MFMA
// against 32 rows; groups of at most 128 rows (decode, one token's heads) use
// 32 so no wave idles.  The key tile keeps S^T + P^T + O^T + Q^T within the
// 512 registers a wave has at one wave per SIMD.
Shape pick_shape(int hd, int rows_per_group) {
  if (hd == 256) return {32, 64};
  if (rows_per_group > 128) return {64, hd == 128 ? 64 : 128};
  return {32, 128};
}

template <int HD, int QW, int KT>
hipError_t launch_t(const FwdParams& p, bool gather, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)p.tiles_per_group * p.n_groups * p.num_splits));
  if (gather)
    hipLaunchKernelGGL((fwd_kernel<HD, QW, KT, true>), grid, dim3(THREADS), 0, stream, p);
  else
    hipLaunchKernelGGL((fwd_kernel<HD, QW, KT, false>), grid, dim3(THREADS), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

int64_t fwd_grid_size(const FwdParams& p, int hd) {
  const Shape sh = pick_shape(hd, p.rows_per_group);
  const int64_t m_wg = (int64_t)WAVES * sh.qw;
  const int64_t tiles = (p.rows_per_group + m_wg - 1) / m_wg;
  return tiles * p.n_groups * p.num_splits;
}

hipError_t launch_fwd(FwdParams p, int hd, hipStream_t stream) {
  const Shape sh = pick_shape(hd, p.rows_per_group);
  const int m_wg = WAVES * sh.qw;
  p.tiles_per_group = (p.rows_per_group + m_wg - 1) / m_wg;
  const bool gather = p.kv_idx != nullptr;
  switch (hd) {
    case 64:
      return sh.qw == 64 ? launch_t<64, 64, 128>(p, gather, stream)
                         : launch_t<64, 32, 128>(p, gather, stream);
    case 128:
      return sh.qw == 64 ? launch_t<128, 64, 64>(p, gather, stream)
                         : launch_t<128, 32, 128>(p, gather, stream);
    case 256:
      return launch_t<256, 32, 64>(p, gather, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace fmha
