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
#include <type_traits>

#include "fmha_device.h"

namespace fmha {
namespace {

using namespace dev;

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

// Streaming kernel: a workgroup takes WAVES*QW rows of one group and walks the
// keys of its split in KT-key tiles, double-buffered in LDS.
template <int HD, int QW, int KT, int WAVES, bool GATHER, int WPE>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void fwd_kernel(FwdParams p) {
  constexpr int THREADS = WAVES * 64;
  constexpr int NQB = QW / 32;
  constexpr int NKB = KT / 32;   // 32-key row blocks of S^T per tile
  constexpr int NKS = KT / 16;   // 16-key contraction steps of PV per tile
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
          (void*)p.k, (short)0, (int)((uint32_t)p.pool_rows * ROW_BYTES), BUF_FLAGS);
      const auto rsv = __builtin_amdgcn_make_buffer_rsrc(
          (void*)p.v, (short)0, (int)((uint32_t)p.pool_rows * ROW_BYTES), BUF_FLAGS);
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
                                                         (short)0, nbytes, BUF_FLAGS);
      const auto rsv = __builtin_amdgcn_make_buffer_rsrc((void*)(vbase + (int64_t)t0 * HD),
                                                         (short)0, nbytes, BUF_FLAGS);
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

  Rows<HD, QW> w;
  w.load_q(p.q, grow0, row0, p.rows_per_group, l32, hlf);
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

    f32x16 s[NKB][NQB];
    w.template qk<NKB>(s, [&](int kb, int ds) {
      return *reinterpret_cast<const bf16x8*>(sb + k_lane + kb * 32 * KS + ds * 32);
    });
    if ((!GATHER && t0 + KT > key_hi) || (GATHER && tile_masked)) {
      w.template mask<NKB>(s, hlf, [&](int kr) {
        return GATHER ? (sValid[buf][kr] != 0) : (t0 + kr < key_hi);
      });
    }
    bf16x8 pf[NQB][NKS];
    if (w.template softmax<NKB>(s, pf, c)) w.rescale_o();
    w.template pv<NKS>(pf, [&](int ks, int db) {
      const char* a = sb + v_lane + 16 * ks * VS + 64 * db;
      return v_frag_tr(a, a + 8 * VS);
    });

    if (have_next) {
      // The other buffer was last read in iteration t-1; every wave has passed
      // the barrier that ended it.
      const int mk = store_tile(buf ^ 1);
      tile_masked = GATHER ? __syncthreads_or(mk) : (__syncthreads(), 0);
    }
  }
  // Epilogue through LDS when this workgroup's output rows fit in the stage
  // buffers (bf16 at hd <= 128), else each lane stores its own pieces.
  constexpr int SMEM_BYTES = 2 * (K_BYTES + V_BYTES);
  constexpr int RB_BF16 = HD * 2;
  if constexpr (WAVES * QW * RB_BF16 <= SMEM_BYTES) {
    if (p.out_mode == OUT_BF16) {
      __syncthreads();
      char* const region = &smem[0][0] + wave * QW * RB_BF16;
      w.store_lds(p, grow0, row0, split, lane, [&](int r) { return region + r * RB_BF16; });
      return;
    }
  }
  w.store(p, grow0, row0, split, l32, hlf);
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
  const int64_t m_wg = (p.chunk <= chunk_max_keys(hd)) ? 128 : (int64_t)sh.waves * sh.qw;
  const int64_t tiles = (p.rows_per_group + m_wg - 1) / m_wg;
  return tiles * p.n_groups * p.num_splits;
}

hipError_t launch_fwd(FwdParams p, int hd, hipStream_t stream) {
  // a split that fits in LDS whole is staged at once (decode shapes)
  if (p.chunk <= chunk_max_keys(hd)) return launch_chunk(p, hd, stream);
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
