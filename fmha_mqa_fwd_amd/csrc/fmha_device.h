// Device-side building blocks shared by the attention kernels (gfx950).
//
// One 32x32x16 bf16 MFMA tile of S^T = K.Q^T holds, in lane l, query column
// l%32 and the 16 keys 8*(r/4) + 4*(l/32) + r%4 (r = accumulator register).
// Every row statistic is therefore in-lane plus one exchange with lane l^32,
// and the bf16-rounded accumulators are, register for register, the B operand
// of the PV MFMA O^T = V^T.P^T when V's A operand lists the keys of each
// 16-key step in the order 8*(e/4) + 4*(l/32) + e%4, e = 0..7.
//
// The steps follow the pages' pipeline (page "CURRENT ISSUE: UMMA FMHA — Full
// Pipeline + Production", "What's working": QK -> softmax -> PV -> output;
// "Key lessons from this session": the scale is applied in the softmax) and the
// multi-KV-tile O rescale (page "May 24, 2026 — Session Start Plan", section 2).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fmha_internal.h"

namespace fmha {
namespace dev {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr float LN2 = 0.6931471805599453f;
// The running max used for the exponentials is left where it is while a
// lane's sum of one tile's exponentials stays at or below this bound: every
// exponential is then <= 2^12, far inside fp32/bf16 range, and O/l need
// rescaling on few tiles.
constexpr float SUM_LIMIT = 4096.0f;
// LDS operand reads issued ahead of their MFMAs (Rows::qk, Rows::pv)
constexpr int QK_DEPTH = 4;
constexpr int PV_DEPTH = 3;
// gfx9 raw buffer descriptor word 3 (32-bit data, no swizzle, offset mode)
constexpr int BUF_FLAGS = 0x00020000;
// Cache-policy operand of the buffer-load builtins: the non-temporal bit
// (data read once; measured ~1% faster for the split-KV decode's K/V).
constexpr int CPOL_NT = 2;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// Two floats to two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

__device__ __forceinline__ bf16x8 pack_bf16x8(const float* s) {
  u32x4 w;
  w[0] = pack_bf16x2(s[0], s[1]);
  w[1] = pack_bf16x2(s[2], s[3]);
  w[2] = pack_bf16x2(s[4], s[5]);
  w[3] = pack_bf16x2(s[6], s[7]);
  return __builtin_bit_cast(bf16x8, w);
}

// Workgroup id -> (row tile, group, split).  The dispatcher hands workgroup
// i to XCD i mod 8, and each XCD has its own L2.  The row tiles of one
// (group, split) unit read the same K/V, so when a unit has a few of them
// (at most 8) they are placed 8 ids apart -- same XCD, same dispatch round --
// and the second reader finds the unit's K/V in that L2.  Units are taken in
// blocks of 8; a last partial block of rem units is laid out tile-major.
// With more than 8 row tiles a unit covers every XCD anyway, and its tiles
// stay consecutive.  A bijection onto [0, tiles) x [0, n_groups * splits).
struct WgCoords {
  int tile, group, split;
};
__device__ __forceinline__ WgCoords wg_coords(int bid, int tiles, int n_groups, int units) {
  int tile, unit;
  if (tiles == 1 || tiles > 8) {
    tile = bid % tiles;
    unit = bid / tiles;
  } else {
    const int full = units & ~7;
    if (bid < full * tiles) {
      const int blk = bid / (8 * tiles), r = bid - blk * 8 * tiles;
      tile = r >> 3;
      unit = blk * 8 + (r & 7);
    } else {
      const int r = bid - full * tiles, rem = units - full;
      tile = r / rem;
      unit = full + r % rem;
    }
  }
  return {tile, unit % n_groups, unit / n_groups};
}

// Value of lane l^32 combined with this lane's: max and sum across the halves.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Attention sink (page "May 24, 2026 — Session Start Plan": a "sink merge" is
// named, its formula is not printed; reading: one extra logit `s` per query
// head whose value vector is zero).  Given a row's normalised output scale
// `inv` and its log-sum-exp `lse` (natural log) over the real keys, the sink
// joins the denominator: lse' = ln(e^lse + e^s) and O' = O e^(lse - lse').
// s = -inf leaves the row as it is; a row without keys gets O = 0, lse' = s.
__device__ __forceinline__ void sink_adjust(float s, float& inv, float& lse) {
  if (s == neg_inf()) return;
  if (lse == neg_inf()) {
    inv = 0.f;
    lse = s;
    return;
  }
  const float hi = fmaxf(lse, s);
  const float l2 = hi + log1pf(expf(-fabsf(lse - s)));
  inv *= expf(lse - l2);
  lse = l2;
}

// Key (within a 32-key block) held by accumulator register r of a lane in half
// `hlf` of the wave (32x32 MFMA output layout).
__device__ __forceinline__ int acc_row(int r, int hlf) { return 8 * (r >> 2) + 4 * hlf + (r & 3); }

// Per-wave state of QW query rows (NQB = QW/32 column blocks) over HD of the
// head dim; LD is the row length of q and of the output (HD, or the full head
// dim when several waves share the rows and each holds a column range).
template <int HD, int QW, int LD = HD>
struct Rows {
  static constexpr int NQB = QW / 32;
  static constexpr int NDS = HD / 16;  // 16-wide contraction steps of QK^T
  static constexpr int NDB = HD / 32;  // 32-wide d blocks of O^T
  bf16x8 qf[NQB][NDS];                 // Q^T fragments (B operand of S^T)
  f32x16 o[NDB][NQB];                  // O^T accumulators
  float m[NQB];                        // running max, scaled, log2 units
  float l[NQB];                        // this lane-half's running row sum
  float alpha[NQB];                    // last rescale factor

  // Lane (hlf, l32) of block qb holds q[row l32][col0 + 16*ds + 8*hlf .. +7].
  __device__ __forceinline__ void load_q(const uint16_t* q, int64_t grow0, int row0,
                                         int rows_in_group, int l32, int hlf, int col0 = 0) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int r = row0 + qb * 32 + l32;
      const bool ok = r < rows_in_group;
      const uint16_t* qrow = q + (grow0 + (ok ? r : 0)) * LD + col0 + 8 * hlf;
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (ok) w = *reinterpret_cast<const u32x4*>(qrow + 16 * ds);
        qf[qb][ds] = __builtin_bit_cast(bf16x8, w);
      }
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][qb][i] = 0.f;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      m[qb] = neg_inf();
      l[qb] = 0.f;
      alpha[qb] = 1.f;
    }
  }

  // The one-block QK^T with mid(ds) run right after the MFMA of step ds: work
  // whose issue then overlaps the matrix unit (the next tile's DMA).  Same
  // MFMA order and result as qk.
  template <class KFrag, class Mid>
  __device__ __forceinline__ void qk_mid(f32x16 (&s)[1][NQB], KFrag kfrag, Mid mid) const {
    static_assert(NQB == 1 && NDS >= QK_DEPTH, "one block");
    constexpr int D = QK_DEPTH;
    bf16x8 a[D];
#pragma unroll
    for (int i = 0; i < D; ++i) a[i] = kfrag(0, i);
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      __builtin_amdgcn_sched_barrier(0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ds % D], qf[0][ds], acc, 0, 0, 0);
      if (ds + D < NDS) a[ds % D] = kfrag(0, ds + D);
      mid(ds);
    }
    __builtin_amdgcn_sched_barrier(0);
    s[0][0] = acc;
  }

  // S^T[kb][qb] = K_tile . Q^T with kfrag(kb, ds) the 16-byte A fragment of
  // key block kb (32 keys) and contraction step ds.
  template <int NKB, class KFrag>
  __device__ __forceinline__ void qk(f32x16 (&s)[NKB][NQB], KFrag kfrag) const {
    // one 32x32 block: the K fragments are read QK_DEPTH steps ahead of
    // their MFMA (the compiler's own order kept two in flight, and each MFMA
    // pair waited on LDS; ~0.5% faster per prefill call), same MFMA order
    if constexpr (NKB == 1 && NQB == 1 && NDS >= QK_DEPTH) {
      constexpr int D = QK_DEPTH;
      bf16x8 a[D];
#pragma unroll
      for (int i = 0; i < D; ++i) a[i] = kfrag(0, i);
      f32x16 acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        __builtin_amdgcn_sched_barrier(0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ds % D], qf[0][ds], acc, 0, 0, 0);
        if (ds + D < NDS) a[ds % D] = kfrag(0, ds + D);
      }
      __builtin_amdgcn_sched_barrier(0);
      s[0][0] = acc;
      return;
    }
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
        const bf16x8 a = kfrag(kb, ds);
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
          s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][ds], s[kb][qb], 0, 0, 0);
      }
    }
  }

  // -inf for the keys of this tile for which key_ok(key within tile) is false.
  template <int NKB, class KeyOk>
  __device__ __forceinline__ void mask(f32x16 (&s)[NKB][NQB], int hlf, KeyOk key_ok) const {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (!key_ok(32 * kb + acc_row(r, hlf))) {
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) s[kb][qb][r] = neg_inf();
        }
      }
  }

  // exp2(s*c - m) of one query block's tile into the bf16 P^T fragments;
  // returns this lane's fp32 sum of the values (before bf16 rounding, so the
  // log-sum-exp keeps fp32 accuracy).
  template <int NKB>
  __device__ __forceinline__ float exps(const f32x16 (&s)[NKB][NQB], bf16x8 (&pf)[NQB][2 * NKB],
                                        int qb, float c, float m_use) const {
    float ls0, ls1;  // the sums start at the first pair (no add of 0)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float a = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][8 * h + 2 * j], c, -m_use));
          const float b = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][8 * h + 2 * j + 1], c, -m_use));
          w[j] = pack_bf16x2(a, b);
          if (kb == 0 && h == 0 && j == 0) {
            ls0 = a;
            ls1 = b;
          } else {
            ls0 += a;
            ls1 += b;
          }
        }
        pf[qb][2 * kb + h] = __builtin_bit_cast(bf16x8, w);
      }
    }
    return ls0 + ls1;
  }

  // S^T of the next tile (one 32x32 block, as qk) with the fast-path
  // exponentials of the current tile (as softmax_fast) spread between its
  // MFMAs: with one wave per SIMD the next tile's matrix work then runs
  // while this wave's vector unit takes the exponentials.  Same operations in
  // the same order per value as qk and softmax_fast, so the same bits; returns
  // softmax_fast's verdict.
  template <class KFrag>
  __device__ __forceinline__ bool qk_next_softmax(f32x16 (&s_next)[1][NQB], KFrag kfrag,
                                                  const f32x16 (&s_cur)[1][NQB],
                                                  bf16x8 (&pf)[NQB][2], float c,
                                                  float (&ls)[NQB]) const {
    static_assert(NQB == 1 && NDS >= QK_DEPTH && 16 % NDS == 0, "one block");
    constexpr int D = QK_DEPTH, PER = 16 / NDS;  // exponentials per MFMA
    bf16x8 a[D];
#pragma unroll
    for (int i = 0; i < D; ++i) a[i] = kfrag(0, i);
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    const float mu = m[0];
    float e[16];
    u32x4 w[2];
    float ls0, ls1;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      __builtin_amdgcn_sched_barrier(0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ds % D], qf[0][ds], acc, 0, 0, 0);
      if (ds + D < NDS) a[ds % D] = kfrag(0, ds + D);
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int j = ds * PER + u;
        e[j] = __builtin_amdgcn_exp2f(fmaf(s_cur[0][0][j], c, -mu));
        // empty asm "writing" each value where it is made: it keeps the
        // compiler from sinking the slice's work below the later MFMAs
        asm volatile("" : "+v"(e[j]));
        if (j & 1) {
          const int k = j >> 1;  // pair k = 4h + i: word i of fragment h
          uint32_t pk = pack_bf16x2(e[j - 1], e[j]);
          asm volatile("" : "+v"(pk));
          w[k >> 2][k & 3] = pk;
          if (k == 0) {
            ls0 = e[0];
            ls1 = e[1];
          } else {
            ls0 += e[j - 1];
            ls1 += e[j];
          }
          asm volatile("" : "+v"(ls0), "+v"(ls1));
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    s_next[0][0] = acc;
    pf[0][0] = __builtin_bit_cast(bf16x8, w[0]);
    pf[0][1] = __builtin_bit_cast(bf16x8, w[1]);
    ls[0] = ls0 + ls1;
    return __any(!(ls[0] <= SUM_LIMIT));
  }

  // Online softmax of one tile in base 2 (x*scale*log2e - m in one FMA), in
  // two halves.  softmax_fast takes the exponentials against the running max
  // as it is and returns (wave-uniform) whether they must be redone: some
  // lane's sum exceeds SUM_LIMIT, or is inf/NaN because there is no max yet.
  // softmax_slow then takes the exact tile max, moves the max, scales l and
  // sets alpha (O must be scaled by it), and redoes the exponentials.  Exact
  // either way: O and l always share the maximum they were computed against.
  // commit_l adds the tile's sums to l.
  template <int NKB>
  __device__ __forceinline__ bool softmax_fast(const f32x16 (&s)[NKB][NQB],
                                               bf16x8 (&pf)[NQB][2 * NKB], float c,
                                               float (&ls)[NQB]) const {
    bool bad = false;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      ls[qb] = exps<NKB>(s, pf, qb, c, m[qb]);
      bad |= !(ls[qb] <= SUM_LIMIT);
    }
    return __any(bad);
  }

  template <int NKB>
  __device__ __forceinline__ void softmax_slow(const f32x16 (&s)[NKB][NQB],
                                               bf16x8 (&pf)[NQB][2 * NKB], float c,
                                               float (&ls)[NQB]) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      float mx = neg_inf();
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
      const float m_new = fmaxf(m[qb], pair_max(mx) * c);
      const float a = (m[qb] == neg_inf()) ? 0.f
                      : (m_new == m[qb])   ? 1.f
                                           : __builtin_amdgcn_exp2f(m[qb] - m_new);
      alpha[qb] = a;
      l[qb] *= a;
      m[qb] = m_new;
      ls[qb] = exps<NKB>(s, pf, qb, c, (m_new == neg_inf()) ? 0.f : m_new);
    }
  }

  __device__ __forceinline__ void commit_l(const float (&ls)[NQB]) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) l[qb] += ls[qb];
  }

  // Both halves in sequence; returns whether O must be scaled by alpha before
  // the next PV.
  template <int NKB>
  __device__ __forceinline__ int softmax(f32x16 (&s)[NKB][NQB], bf16x8 (&pf)[NQB][2 * NKB],
                                         float c) {
    float ls[NQB];
    if (!softmax_fast<NKB>(s, pf, c, ls)) {
      commit_l(ls);
      return 0;
    }
    softmax_slow<NKB>(s, pf, c, ls);
    commit_l(ls);
    return 1;
  }

  __device__ __forceinline__ void rescale_o() {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][qb][i] *= alpha[qb];
  }

  // O^T += V^T . P^T with vfrag(ks, db) the A fragment of 16-key step ks and
  // d block db (keys in the accumulator order described above).
  template <int NKS, class VFrag>
  __device__ __forceinline__ void pv(const bf16x8 (&pf)[NQB][NKS], VFrag vfrag) {
    // the same for V: fragments PV_DEPTH MFMAs ahead, the MFMAs in (ks, db) order
    if constexpr (NQB == 1 && NKS * NDB >= PV_DEPTH) {
      constexpr int N = NKS * NDB, D = PV_DEPTH;
      bf16x8 a[D];
#pragma unroll
      for (int i = 0; i < D; ++i) a[i] = vfrag(i / NDB, i % NDB);
#pragma unroll
      for (int i = 0; i < N; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        o[i % NDB][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i % D], pf[0][i / NDB],
                                                                o[i % NDB][0], 0, 0, 0);
        if (i + D < N) a[i % D] = vfrag((i + D) / NDB, (i + D) % NDB);
      }
      __builtin_amdgcn_sched_barrier(0);
      return;
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const bf16x8 a = vfrag(ks, db);
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
          o[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[qb][ks], o[db][qb], 0, 0, 0);
      }
    }
  }

  // pv with mid(i) run right after its i-th MFMA (the pipelined order above).
  template <int NKS, class VFrag, class Mid>
  __device__ __forceinline__ void pv_mid(const bf16x8 (&pf)[NQB][NKS], VFrag vfrag, Mid mid) {
    static_assert(NQB == 1 && NKS * NDB >= PV_DEPTH, "one block");
    constexpr int N = NKS * NDB, D = PV_DEPTH;
    bf16x8 a[D];
#pragma unroll
    for (int i = 0; i < D; ++i) a[i] = vfrag(i / NDB, i % NDB);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      o[i % NDB][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i % D], pf[0][i / NDB],
                                                              o[i % NDB][0], 0, 0, 0);
      if (i + D < N) a[i % D] = vfrag((i + D) / NDB, (i + D) % NDB);
      mid(i);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // O / l and lse = (m + log2 l) ln 2; an empty row (no key seen) gets O = 0,
  // lse = -inf.  Partial modes write plane `split` of [splits, rows, HD].
  // Direct form: each lane stores its own 4-element pieces (a row's 32-wide d
  // block arrives as 8 pieces from 2 lanes per instruction).
  // col0: first output column this wave holds; write_lse: this wave writes
  // the rows' lse (one wave per row when several share it).  Plain stores:
  // pieces of 16 bytes or less from 32 rows per instruction need the caches
  // to merge them into whole lines (non-temporal stores made such a launch
  // half again as slow).
  __device__ __forceinline__ void store(const FwdParams& p, int64_t grow0, int row0, int split,
                                        int l32, int hlf, int col0 = 0,
                                        bool write_lse = true) const {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const float lt = pair_sum(l[qb]);
      const bool empty = (m[qb] == neg_inf());
      float inv = empty ? 0.f : 1.f / lt;
      float lse_v = empty ? neg_inf() : (m[qb] + log2f(lt)) * LN2;
      const int r = row0 + qb * 32 + l32;
      if (r >= p.rows_per_group) continue;
      const int64_t row = grow0 + r;
      if (p.sink != nullptr && !is_partial(p.out_mode))
        sink_adjust(p.sink[row % p.n_heads], inv, lse_v);
      const int64_t base = is_partial(p.out_mode) ? (int64_t)split * p.total_rows : 0;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int d = 32 * db + 8 * rg + 4 * hlf;
          f32x4 val;
#pragma unroll
          for (int i = 0; i < 4; ++i) val[i] = o[db][qb][4 * rg + i] * inv;
          if (is_bf16(p.out_mode)) {
            u32x2 w = {pack_bf16x2(val[0], val[1]), pack_bf16x2(val[2], val[3])};
            *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.out) + (base + row) * LD + col0 +
                                      d) = w;
          } else {
            *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + (base + row) * LD + col0 + d) =
                val;
          }
        }
      }
      if (hlf == 0 && write_lse) p.lse[base + row] = lse_v;
    }
  }

  // Same result, staged through LDS so that memory sees whole output rows:
  // the wave writes its 32 rows (per column block) into LDS, 16-byte chunks
  // XOR-swizzled by row, then consecutive lanes store consecutive 16-byte
  // chunks of each row.  Those stores are non-temporal: the output is written
  // once and not read again by the kernel, so no cache keeps a place for it
  // (measured 1-3% faster per call, most in the split-KV decode, whose bf16
  // partials are half its traffic).  row_addr(r) is the LDS byte address of local row r
  // (0..31), holding at least HD*4 bytes; only this wave touches it.
  template <class RowAddr>
  __device__ __forceinline__ void store_lds(const FwdParams& p, int64_t grow0, int row0, int split,
                                            int lane, RowAddr row_addr, int col0 = 0,
                                            bool write_lse = true) const {
    const int l32 = lane & 31;
    const int hlf = lane >> 5;
    const bool bf = is_bf16(p.out_mode);
    const int esz = bf ? 2 : 4;
    const int rb = HD * esz;            // bytes of a row this wave holds
    const int64_t grb = (int64_t)LD * esz;  // bytes of a whole output row
    const int cpr = rb / 16;            // 16-byte chunks per row (8 .. 64)
    const int swm = cpr >= 16 ? 15 : 7;
    const int64_t base = is_partial(p.out_mode) ? (int64_t)split * p.total_rows : 0;
    char* const out = static_cast<char*>(p.out);
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const float lt = pair_sum(l[qb]);
      const bool empty = (m[qb] == neg_inf());
      float inv = empty ? 0.f : 1.f / lt;
      float lse_v = empty ? neg_inf() : (m[qb] + log2f(lt)) * LN2;
      if (p.sink != nullptr && !is_partial(p.out_mode)) {
        const int rs = row0 + qb * 32 + l32;
        if (rs < p.rows_per_group) sink_adjust(p.sink[(grow0 + rs) % p.n_heads], inv, lse_v);
      }
      char* const my = row_addr(l32);
      const int sw = l32 & swm;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int d = 32 * db + 8 * rg + 4 * hlf;
          f32x4 val;
#pragma unroll
          for (int i = 0; i < 4; ++i) val[i] = o[db][qb][4 * rg + i] * inv;
          if (bf) {
            const u32x2 w = {pack_bf16x2(val[0], val[1]), pack_bf16x2(val[2], val[3])};
            *reinterpret_cast<u32x2*>(my + 16 * ((d >> 3) ^ sw) + 2 * (d & 7)) = w;
          } else {
            *reinterpret_cast<f32x4*>(my + 16 * ((d >> 2) ^ sw)) = val;
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int rpi = 64 / cpr;  // rows per store instruction
      for (int r = lane / cpr; r < 32; r += rpi) {
        const int ch = lane % cpr;
        const u32x4 v = *reinterpret_cast<const u32x4*>(row_addr(r) + 16 * (ch ^ (r & swm)));
        const int rr = row0 + qb * 32 + r;
        if (rr < p.rows_per_group)
          __builtin_nontemporal_store(
              v, reinterpret_cast<u32x4*>(out + (base + grow0 + rr) * grb + col0 * esz + 16 * ch));
      }
      const int r = row0 + qb * 32 + l32;
      if (hlf == 0 && write_lse && r < p.rows_per_group) p.lse[base + grow0 + r] = lse_v;
      __builtin_amdgcn_wave_barrier();  // LDS reads done before the next block's writes
    }
  }
};

// ---- K/V movement by LDS-DMA (buffer_load_dwordx4 ... lds): each lane's 16
// bytes land at M0 + 16*lane in LDS, no registers involved.

constexpr uint32_t OOB = 0x80000000u;  // beyond any descriptor's byte count: reads zeros

// One LDS-DMA instruction from inline assembly: the compiler tracks none of
// these, so it inserts no completion waits of its own; the kernels wait with
// wait_vmcnt.  M0 (the LDS destination) is the asm operand bound to m0.
__device__ __forceinline__ void dma16(u32x4 rsrc, uint32_t lds_addr, uint32_t voff) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "{m0}"(lds_addr), "v"(voff), "s"(rsrc)
               : "memory");
}

// The same, non-temporal (data read once).
__device__ __forceinline__ void dma16_nt(u32x4 rsrc, uint32_t lds_addr, uint32_t voff) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
               :
               : "{m0}"(lds_addr), "v"(voff), "s"(rsrc)
               : "memory");
}

// Raw buffer descriptor over [base, base + nbytes): reads past the end return zeros.
__device__ __forceinline__ u32x4 buffer_rsrc(const void* base, uint32_t nbytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
  r[2] = __builtin_amdgcn_readfirstlane(nbytes);
  r[3] = BUF_FLAGS;
  return r;
}

// s_waitcnt vmcnt(N) with the other counters left unconstrained (gfx9
// encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] in [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// XOR swizzles of 16-byte chunks in unpadded LDS rows of CPR chunks: K uses
// chunk ^ swz_k(row) so that the 16 rows one operand read touches at a column
// land on distinct banks; V uses chunk ^ swz_v(row) for the 4-row x 64-byte
// footprint of ds_read_b64_tr_b16.
template <int CPR>
__device__ __forceinline__ int swz_k(int row) {
  if constexpr (CPR >= 16) return row & 15;
  else return (row & 7) ^ ((row >> 3) & 1);
}
template <int CPR>
__device__ __forceinline__ int swz_v(int row) {
  if constexpr (CPR >= 16) return (0xCA60 >> (4 * (row & 3))) & 15;  // 0, 6, 10, 12
  else return (0x2460 >> (4 * (row & 3))) & 15;                      // 0, 6, 4, 2
}

// ---- Order of a gathered key list.  Attention does not depend on the order
// of its keys, so a split's list may be walked in any order.  Walked by pool
// region, the workgroups that run at one time on an XCD read rows from the same
// part of the pool and share that XCD's L2 lines; walked in list order (a
// uniform draw) they read rows from all of it.

// Region class of a list entry: row >> shift over 32 regions of the pool for
// a usable row, 32 for an entry that reads nothing (it goes last).
__device__ __forceinline__ int region_shift(int pool_rows) {
  const int bits = pool_rows > 1 ? 32 - __clz(pool_rows - 1) : 0;  // ceil(log2(pool_rows))
  return bits > 5 ? bits - 5 : 0;
}
constexpr int REGION_NONE = 32;
// Lists of fewer tiles are walked as given: a decode split of a few tiles
// gains nothing from the order and its one-round launch pays the sort's
// time in full (measured: two-source decode 28.8 us with its 4-tile splits
// sorted, 27.7 us without).
constexpr int ORDER_MIN_TILES = 8;

// Stable counting sort of a list of up to 64 * WAVES * SLOTS entries by region
// class.  Entry i (i < n) is held by lane i % 64 of wave (i / 64) % WAVES in
// slot (i / 64) / WAVES as (off, cls); it is stored to dst at its position in
// the ordered list (equal classes keep their list order, so the order, and the
// kernel's result, are the same on every run).  cnt is LDS scratch of
// 64 * WAVES * SLOTS ints.  Two workgroup barriers; the caller's barrier must
// follow before dst is read.  Returns the number of usable entries: they are
// dst[0 .. n_usable - 1], the unusable ones after them.
template <int WAVES, int SLOTS>
__device__ __forceinline__ int order_by_region(const uint32_t (&off)[SLOTS],
                                               const int (&cls)[SLOTS], int n, uint32_t* dst,
                                               int* cnt, int wave, int lane) {
  constexpr int NCH = WAVES * SLOTS;  // 64-entry chunks
  int rank[SLOTS];
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const int ch = wave + WAVES * s;
    const bool present = 64 * ch + lane < n;
    uint64_t own = __ballot(present);  // lanes of this chunk in my class
    uint64_t of_lane = own;            // lanes of this chunk in class `lane`
#pragma unroll
    for (int b = 0; b < 6; ++b) {
      // lanes whose class has bit b set; kept against per-lane flips (a
      // per-lane choice between the mask and its complement keeps both in
      // scalar registers, and the slots' pairs spilled)
      const uint64_t bb = __ballot(present && ((cls[s] >> b) & 1));
      own &= bb ^ (((cls[s] >> b) & 1) ? 0ull : ~0ull);
      of_lane &= bb ^ (((lane >> b) & 1) ? 0ull : ~0ull);
    }
    rank[s] = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(own >> 32),
                                             __builtin_amdgcn_mbcnt_lo((uint32_t)own, 0u));
    cnt[64 * ch + lane] = __popcll(of_lane);
    // one slot's masks at a time (interleaved, the slots' ballots spill SGPRs)
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();
  if (wave == 0) {
    // lane = class: each chunk's first position for the class, in class-major
    // then chunk order
    int v[NCH];
    int tot = 0;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      v[ch] = cnt[64 * ch + lane];
      tot += v[ch];
    }
    int x = tot;  // inclusive scan over the 64 classes
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(x, d);
      if (lane >= d) x += y;
    }
    int run = x - tot;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      cnt[64 * ch + lane] = run;
      run += v[ch];
    }
  }
  __syncthreads();
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    const int ch = wave + WAVES * s;
    if (64 * ch + lane < n) dst[cnt[64 * ch + cls[s]] + rank[s]] = off[s];
  }
  return cnt[REGION_NONE];  // chunk 0's first position of the unusable class
}

// A V fragment from two ds_read_b64_tr_b16 reads at byte addresses a0 (keys
// e = 0..3) and a1 (keys e = 4..7) within LDS.
__device__ __forceinline__ bf16x8 v_frag_tr(const char* a0, const char* a1) {
  const i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)a0);
  const i16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)a1);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
}

}  // namespace dev
}  // namespace fmha
