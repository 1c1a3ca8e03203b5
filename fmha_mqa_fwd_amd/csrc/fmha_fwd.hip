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
//   * keys processed tile by tile with the running O rescaled when the row
//     maximum grows (same page, 2 "Test O Rescale at s_k > 128");
//   * O and the row log-sum-exp as outputs (same page, "D1 Status Summary");
//   * optional row gather of the s_k = top_k selected keys from a KV pool (same
//     page "Key Numbers"; dsv4/kernels/cuda commit log, KV row gather).
//
// How it is mapped onto CDNA4 (our design, not the pages' Blackwell one):
//   * Head-packed M: the rows of a group (all (t, h) of a batch, or all heads of
//     a token) share K/V, so a workgroup takes WAVES*QW consecutive rows and
//     every K/V tile staged in LDS serves all of them.
//   * S^T = K . Q^T with v_mfma_f32_32x32x16_bf16: K (A operand) from LDS, Q^T
//     (B operand) in VGPRs for the whole kernel.  In the 32x32 accumulator
//     layout lane l holds query column l%32 and 16 of the 32 keys, so a row's
//     max/sum is an in-lane reduction plus one v_permlane32_swap, and the
//     per-row rescale factor is a per-lane scalar.
//   * O^T = V^T . P^T: the S^T accumulators, rounded to bf16, are the B operand
//     of the PV MFMA as they stand (P never leaves registers).  V stays
//     row-major in LDS; its A operand is read with ds_read_b64_tr_b16, whose
//     16-lane transpose yields, for lane (d, half h), the keys that lane half h
//     holds in S^T — in the same order.
//   * Online softmax in base 2: x*scale*log2(e) folded into one FMA, exp2 on the
//     transcendental unit, and a lazy rescale: the running maximum used for the
//     exponentials only moves when a row's maximum grows by more than 2^8, so
//     O and l are rescaled on a few tiles instead of every tile (exact: O and l
//     always share the maximum they were computed against).
//   * K/V tiles are double-buffered in LDS; the next tile's global loads are
//     issued into registers before the current tile's MFMAs and written to the
//     other buffer after them, so one barrier per tile suffices and load
//     latency hides behind compute.  Two workgroups share a CU where registers
//     allow, so one wave's softmax overlaps another's MFMAs.
//   * LDS rows use XOR swizzles of 16-byte chunks chosen so that the MFMA operand
//     reads and the staging writes are free of bank conflicts.
#include <math.h>

#include "fmha_internal.h"

namespace fmha {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr float LN2 = 0.6931471805599453f;
// The running max moves only when a row max exceeds it by more than this
// (log2 units): exponentials then stay <= 2^8, far inside fp32/bf16 range.
constexpr float RESCALE_THRESHOLD = 8.0f;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// LDS row strides (bytes).  K rows are read as ds_read_b128 by 16 lanes at 16
// consecutive rows and one column: a 16-byte pad puts those rows on 16
// distinct bank groups.  V rows are read by ds_read_b64_tr_b16, where the 32
// lanes of a wave half read 4 consecutive rows x 64 bytes: a 64-byte pad puts
// the 4 rows on disjoint bank ranges.  Padding (not an XOR swizzle) keeps every
// operand address a per-lane base plus a compile-time offset.
template <int HD>
struct Lds {
  static constexpr int K_STRIDE = HD * 2 + 16;
  static constexpr int V_STRIDE = HD * 2 + 64;
};

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

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

// Value of lane l^32 combined with this lane's: max and sum across the halves.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Key (within a 32-key block) held by accumulator register r of a lane in
// half `hlf`, for the 32x32 MFMA output layout: register r covers row
// 8*(r/4) + 4*hlf + r%4 at column lane%32.
__device__ __forceinline__ int acc_row(int r, int hlf) {
  return 8 * (r >> 2) + 4 * hlf + (r & 3);
}

template <int HD, int QW, int KT, int WAVES, bool GATHER, int WPE>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void fwd_kernel(FwdParams p) {
  constexpr int THREADS = WAVES * 64;
  constexpr int NQB = QW / 32;   // 32-query MFMA column blocks per wave
  constexpr int NDS = HD / 16;   // 16-wide contraction steps of QK^T
  constexpr int NKB = KT / 32;   // 32-key row blocks of S^T per tile
  constexpr int NKS = KT / 16;   // 16-key contraction steps of PV per tile
  constexpr int NDB = HD / 32;   // 32-wide d blocks of O^T
  constexpr int CPR = HD / 8;    // 16-byte chunks per K/V row
  constexpr int M_WG = WAVES * QW;
  constexpr int TILE_CH = KT * CPR;            // chunks per K (or V) tile
  constexpr int CPT = TILE_CH / THREADS;       // chunks per thread per tile
  constexpr int ROWS_PER_PASS = THREADS / CPR;
  constexpr int KS = Lds<HD>::K_STRIDE;
  constexpr int VS = Lds<HD>::V_STRIDE;
  constexpr int K_BYTES = KT * KS;
  constexpr int V_BYTES = KT * VS;
  static_assert(QW % 32 == 0 && KT % 32 == 0 && HD % 32 == 0, "tile shape");
  static_assert(TILE_CH % THREADS == 0 && THREADS % CPR == 0, "staging shape");

  // [buf][K tile | V tile], padded rows
  __shared__ __attribute__((aligned(16))) char smem[2][K_BYTES + V_BYTES];
  __shared__ int sValid[GATHER ? 2 : 1][KT];

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
  const int n_tiles = key_hi > key_lo ? (key_hi - key_lo + KT - 1) / KT : 0;
  const int row0 = tile * M_WG + wave * QW;  // first row of this wave in its group
  const int64_t grow0 = (int64_t)group * p.rows_per_group;
  const uint16_t* kbase = GATHER ? p.k : p.k + (int64_t)group * p.s_k * HD;
  const uint16_t* vbase = GATHER ? p.v : p.v + (int64_t)group * p.s_k * HD;
  const int32_t* ibase = GATHER ? p.kv_idx + (int64_t)group * p.s_k : nullptr;

  // Staging assignment: chunk `sc` of tile rows srow0 + ROWS_PER_PASS*i.
  const int sc = tid % CPR;
  const int srow0 = tid / CPR;

  // ---- staging: global -> registers -> LDS, through buffer loads.  A buffer
  // load whose offset lies beyond the descriptor's byte count returns zeros,
  // which is how keys past the end of this split (dense) or with an
  // out-of-range pool row (gather) become zero rows without predication.
  u32x4 rk[CPT], rv[CPT];
  int ridx[CPT];   // gather: pool rows of the tile being loaded (-1 = masked)
  int rvalid[CPT];
  constexpr uint32_t ROW_BYTES = HD * 2;
  constexpr uint32_t OOB = 0x80000000u;  // beyond any descriptor's byte count
  // Gather: pool-row indices of tile t (read one tile ahead of its K/V).
  auto load_idx = [&](int t) {
    const int t0 = key_lo + t * KT;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int key = t0 + srow0 + ROWS_PER_PASS * i;
      ridx[i] = key < key_hi ? ibase[key] : -1;
    }
  };
  auto load_tile = [&](int t) {
    const int t0 = key_lo + t * KT;
    if constexpr (GATHER) {
      const auto rsk = __builtin_amdgcn_make_buffer_rsrc(
          (void*)p.k, (short)0, (int)((uint32_t)p.pool_rows * ROW_BYTES), 0x00020000);
      const auto rsv = __builtin_amdgcn_make_buffer_rsrc(
          (void*)p.v, (short)0, (int)((uint32_t)p.pool_rows * ROW_BYTES), 0x00020000);
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int idx = ridx[i];
        const bool ok = idx >= 0 && idx < p.pool_rows;
        rvalid[i] = ok;
        const uint32_t off = ok ? (uint32_t)idx * ROW_BYTES + 16 * sc : OOB;
        rk[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsk, off, 0, 0));
        rv[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsv, off, 0, 0));
      }
    } else {
      // descriptor covers keys t0 .. key_hi-1 of this group
      const int nbytes = (key_hi - t0) * (int)ROW_BYTES;
      const auto rsk = __builtin_amdgcn_make_buffer_rsrc((void*)(kbase + (int64_t)t0 * HD),
                                                         (short)0, nbytes, 0x00020000);
      const auto rsv = __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + (int64_t)t0 * HD),
                                                         (short)0, nbytes, 0x00020000);
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const uint32_t off = (uint32_t)(srow0 + ROWS_PER_PASS * i) * ROW_BYTES + 16 * sc;
        rk[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsk, off, 0, 0));
        rv[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsv, off, 0, 0));
        rvalid[i] = 1;
      }
    }
  };
  // Returns nonzero when this thread staged a masked key (gather only).
  auto store_tile = [&](int buf) {
    int masked = 0;
    char* sk = smem[buf];
    char* sv = smem[buf] + K_BYTES;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int row = srow0 + ROWS_PER_PASS * i;
      *reinterpret_cast<u32x4*>(sk + row * KS + 16 * sc) = rk[i];
      *reinterpret_cast<u32x4*>(sv + row * VS + 16 * sc) = rv[i];
      if constexpr (GATHER) {
        if (sc == 0) sValid[buf][row] = rvalid[i];
        masked |= !rvalid[i];
      }
    }
    return masked;
  };

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
  float m[NQB], l[NQB];  // running max (scaled, log2 units) and partial row sum
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    m[qb] = neg_inf();
    l[qb] = 0.f;
  }
  const float c = p.scale_log2;

  // Per-lane LDS byte offsets of the MFMA operands within a stage buffer.
  //  K (A of S^T, ds_read_b128): row 32*kb + l32, bytes 32*ds + 16*hlf.
  //  V (A of O^T, ds_read_b64_tr_b16): lane (jj, dsub, hlf) of K-step ks,
  //  d block db and half r reads row 16*ks + 8*r + 4*hlf + jj/4, columns
  //  32*db + 16*dsub + 4*(jj%4) .. +3; the 16-lane transpose then hands lane
  //  (d = 32*db + lane%32, hlf) the keys 16*ks + 8*(e/4) + 4*hlf + e%4, e = 0..7,
  //  which is where S^T's accumulator layout put that lane's P values.
  const int jj = lane & 15;
  const int dsub = (lane >> 4) & 1;
  const int k_lane = l32 * KS + 16 * hlf;
  const int v_lane = K_BYTES + (4 * hlf + (jj >> 2)) * VS + 2 * (16 * dsub + 4 * (jj & 3));

  int tile_masked = 0;
  if (n_tiles > 0) {
    if constexpr (GATHER) load_idx(0);
    load_tile(0);
    if constexpr (GATHER) {
      if (n_tiles > 1) load_idx(1);
    }
    const int mk = store_tile(0);
    tile_masked = GATHER ? __syncthreads_or(mk) : (__syncthreads(), 0);
  }

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    const int t0 = key_lo + t * KT;
    const bool have_next = t + 1 < n_tiles;
    if (have_next) {
      load_tile(t + 1);
      if constexpr (GATHER) {
        if (t + 2 < n_tiles) load_idx(t + 2);
      }
    }
    const char* sb = smem[buf];

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
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(sb + k_lane + kb * 32 * KS + ds * 32);
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
          s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][ds], s[kb][qb], 0, 0, 0);
      }
    }
    const bool dense_tail = !GATHER && (t0 + KT > key_hi);
    if (dense_tail || (GATHER && tile_masked)) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kr = 32 * kb + acc_row(r, hlf);
          const bool ok = GATHER ? (sValid[buf][kr] != 0) : (t0 + kr < key_hi);
          if (!ok) {
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) s[kb][qb][r] = neg_inf();
          }
        }
    }

    // ---- online softmax (base 2) with lazy rescale
    bf16x8 pf[NQB][NKS];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      float mx = neg_inf();
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
      const float m_tile = pair_max(mx) * c;
      if (__any(m_tile > m[qb] + RESCALE_THRESHOLD)) {
        const float m_new = fmaxf(m[qb], m_tile);
        const float m_old_use = (m[qb] == neg_inf()) ? m_new : m[qb];
        const float alpha = (m_new == neg_inf()) ? 1.f : __builtin_amdgcn_exp2f(m_old_use - m_new);
        const float a0 = (m[qb] == neg_inf()) ? 0.f : alpha;
        l[qb] *= a0;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[db][qb][i] *= a0;
        m[qb] = m_new;
      }
      const float m_use = (m[qb] == neg_inf()) ? 0.f : m[qb];
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
      l[qb] += ls;
    }

    // ---- O^T += V^T . P^T
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        i16x4 part[2];
#pragma unroll
        for (int r = 0; r < 2; ++r)
          part[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(sb + v_lane + (16 * ks + 8 * r) * VS + 64 * db));
        const bf16x8 a = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
          o[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[qb][ks], o[db][qb], 0, 0, 0);
      }
    }

    if (have_next) {
      // The other buffer was last read in iteration t-1; every wave has passed
      // the barrier that ended it.
      const int mk = store_tile(buf ^ 1);
      tile_masked = GATHER ? __syncthreads_or(mk) : (__syncthreads(), 0);
    }
  }

  // ---- epilogue: O / l, lse = (m + log2 l) * ln 2
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const float lt = pair_sum(l[qb]);
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
  int qw, kt, waves, wpe;
};

// 32 rows per wave keeps a wave within 170 (dense, 32-key tiles: three waves
// per SIMD) or 256 (gather, 64-key tiles: two waves per SIMD) registers, so
// one wave's softmax overlaps other waves' MFMAs.  hd 256 needs the whole
// register file: one wave per SIMD.
Shape pick_shape(int hd, bool gather) {
  if (hd == 256) return {32, 32, 4, 1};
  if (gather) return {32, 64, 4, 2};
  return {32, 32, 4, 3};
}

template <int HD, int QW, int KT, int WAVES, int WPE, bool GATHER>
hipError_t launch_t(const FwdParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)p.tiles_per_group * p.n_groups * p.num_splits));
  hipLaunchKernelGGL((fwd_kernel<HD, QW, KT, WAVES, GATHER, WPE>), grid, dim3(WAVES * 64), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace

int64_t fwd_grid_size(const FwdParams& p, int hd) {
  const Shape sh = pick_shape(hd, p.kv_idx != nullptr);
  const int64_t m_wg = (int64_t)sh.waves * sh.qw;
  const int64_t tiles = (p.rows_per_group + m_wg - 1) / m_wg;
  return tiles * p.n_groups * p.num_splits;
}

hipError_t launch_fwd(FwdParams p, int hd, hipStream_t stream) {
  const bool gather = p.kv_idx != nullptr;
  const Shape sh = pick_shape(hd, gather);
  const int m_wg = sh.waves * sh.qw;
  p.tiles_per_group = (p.rows_per_group + m_wg - 1) / m_wg;
  switch (hd) {
    case 64:
      return gather ? launch_t<64, 32, 64, 4, 2, true>(p, stream)
                    : launch_t<64, 32, 32, 4, 3, false>(p, stream);
    case 128:
      return gather ? launch_t<128, 32, 64, 4, 2, true>(p, stream)
                    : launch_t<128, 32, 32, 4, 3, false>(p, stream);
    case 256:
      return gather ? launch_t<256, 32, 32, 4, 1, true>(p, stream)
                    : launch_t<256, 32, 32, 4, 1, false>(p, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace fmha
