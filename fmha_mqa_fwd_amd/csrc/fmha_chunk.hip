// Multi-query attention forward, whole-chunk variant, for gfx950.
//
// Used when the keys one workgroup attends to (one split of s_k, or all of
// them) fit in LDS at once: 128 keys at hd 256, 256 at hd 128, 512 at hd 64.
// That is the split-KV decode shape (many splits of a short key range, one
// token's query heads per workgroup) that the pages' "Key Numbers" describe
// (Pro decode: 128 heads, top_k 1024 in 8 KV tiles) and the split-KV + merge
// plan of page "CURRENT ISSUE: UMMA FMHA — Full Pipeline + Production", "Next
// steps" item 4.
//
// A decode workgroup does little arithmetic per byte, so its time is the HBM
// latency and bandwidth of its K/V chunk.  The kernel therefore issues the
// whole chunk at once with LDS-DMA buffer loads (buffer_load_dwordx4 ... lds:
// no registers, no VALU) in tile order, then processes tile t as soon as this
// wave's loads up to tile t have landed (s_waitcnt vmcnt) and a barrier has
// published every wave's share.  The attention arithmetic per tile is the same
// as the streaming kernel's (fmha_device.h).
//
// LDS rows are unpadded (DMA writes 1 KiB contiguous per instruction) and
// XOR-swizzled on 16-byte chunks: each lane DMAs the global chunk that belongs
// at its LDS position.  K uses chunk ^ (row & 15) so the 16 rows an operand
// read touches at one column land on distinct banks; V uses chunk ^ {0,6,10,12}
// [row & 3] for the 4-row x 64-byte footprint of ds_read_b64_tr_b16.
#include <type_traits>

#include "fmha_device.h"

namespace fmha {
namespace {

using namespace dev;

constexpr int CHUNK_LDS_BYTES = 64 * 1024;  // per tensor

template <int HD>
struct ChunkShape {
  static constexpr int ROW = HD * 2;                    // bytes per K/V row
  static constexpr int MAXK = CHUNK_LDS_BYTES / ROW;    // keys that fit
};

// Four DMA groups per tensor, each its own LDS object: the compiler waits for
// LDS-DMA completion per LDS object, so separate objects keep its waits at
// group granularity (the kernel's own waits are per group too).
constexpr int NGROUP = 4;  // the wait switch below assumes 4

template <int HD, bool GATHER>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void chunk_kernel(FwdParams p) {
  constexpr int WAVES = 4, QW = 32, KT = 32;
  constexpr int NQB = QW / 32;
  constexpr int ROW = ChunkShape<HD>::ROW;
  constexpr int MAXK = ChunkShape<HD>::MAXK;
  constexpr int GK = MAXK / NGROUP;                // keys per DMA group
  constexpr int TPG = GK / KT;                     // compute tiles per group
  constexpr int CPR = HD / 8;
  constexpr int GROUP_BYTES = GK * ROW;            // 16 KiB
  constexpr int IPW = GROUP_BYTES / 1024 / WAVES;  // DMA instructions per wave, group, tensor
  constexpr int NKS = KT / 16;
  constexpr int M_WG = WAVES * QW;
  static_assert(IPW >= 1 && GROUP_BYTES % (1024 * WAVES) == 0, "DMA shape");
  static_assert(2 * IPW * (NGROUP - 1) < 64, "vmcnt range");

  __shared__ __attribute__((aligned(16))) char sK0[GROUP_BYTES], sK1[GROUP_BYTES],
      sK2[GROUP_BYTES], sK3[GROUP_BYTES];
  __shared__ __attribute__((aligned(16))) char sV0[GROUP_BYTES], sV1[GROUP_BYTES],
      sV2[GROUP_BYTES], sV3[GROUP_BYTES];
  __shared__ int sValid[GATHER ? MAXK : 1];
  auto kgrp = [&](int g) __attribute__((always_inline)) -> char* {
    return g == 0 ? sK0 : g == 1 ? sK1 : g == 2 ? sK2 : sK3;
  };
  auto vgrp = [&](int g) __attribute__((always_inline)) -> char* {
    return g == 0 ? sV0 : g == 1 ? sV1 : g == 2 ? sV2 : sV3;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: DMA guards and M0
  const int l32 = lane & 31;
  const int hlf = lane >> 5;

  const WgCoords wc =
      wg_coords(blockIdx.x, p.tiles_per_group, p.n_groups, p.n_groups * p.num_splits);
  const int tile = wc.tile, group = wc.group, split = wc.split;

  const int key_lo = split * p.chunk;
  const int key_hi = min(key_lo + p.chunk, p.s_k);
  const int nk = max(key_hi - key_lo, 0);  // <= MAXK (host guarantees)
  const int n_tiles = (nk + KT - 1) / KT;
  const int row0 = tile * M_WG + wave * QW;
  const int64_t grow0 = (int64_t)group * p.rows_per_group;

  Rows<HD, QW> w;

  // Lane `lane` of DMA instruction j of group g fills LDS byte
  // inst*1024 + 16*lane of that group, inst = wave*IPW + j: key row
  // g*GK + pos/ROW, physical chunk (pos%ROW)/16.
  auto dma_row = [&](int g, int j) __attribute__((always_inline)) {
    return g * GK + ((wave * IPW + j) * 1024 + lane * 16) / ROW;
  };
  auto dma_phys = [&](int j) __attribute__((always_inline)) {
    return (((wave * IPW + j) * 1024 + lane * 16) % ROW) / 16;
  };

  // ---- gather: pool rows of every key this lane moves (loads first, uses later)
  int gidx[GATHER ? NGROUP * IPW : 1];
  if constexpr (GATHER) {
    const int32_t* ibase = p.kv_idx + (int64_t)group * p.s_k + key_lo;
#pragma unroll
    for (int g = 0; g < NGROUP; ++g)
#pragma unroll
      for (int j = 0; j < IPW; ++j) {
        const int row = dma_row(g, j);
        gidx[g * IPW + j] = row < nk ? ibase[row] : -1;
      }
  }
  // Q next: it is waited for by the first group's wait below.
  w.load_q(p.q, grow0, row0, p.rows_per_group, l32, hlf);
  if constexpr (GATHER) {
#pragma unroll
    for (int i = 0; i < NGROUP * IPW; ++i) {
      const int idx = gidx[i];
      gidx[i] = (idx >= 0 && idx < p.pool_rows) ? idx : -1;
      if (dma_phys(i % IPW) == 0) sValid[dma_row(i / IPW, i % IPW)] = gidx[i] >= 0;
    }
  }

  // ---- issue the whole chunk.  All groups are issued (keys past the split's
  // end read zeros from beyond the descriptor and cost no memory traffic), so
  // every wait count below is a compile-time constant.
  {
    __amdgpu_buffer_rsrc_t rk, rv;
    if constexpr (GATHER) {
      rk = __builtin_amdgcn_make_buffer_rsrc((void*)p.k, (short)0, p.pool_rows * ROW, BUF_FLAGS);
      rv = __builtin_amdgcn_make_buffer_rsrc((void*)p.v, (short)0, p.pool_rows * ROW, BUF_FLAGS);
    } else {
      const int64_t base = ((int64_t)group * p.s_k + key_lo) * HD;
      rk = __builtin_amdgcn_make_buffer_rsrc((void*)(p.k + base), (short)0, nk * ROW, BUF_FLAGS);
      rv = __builtin_amdgcn_make_buffer_rsrc((void*)(p.v + base), (short)0, nk * ROW, BUF_FLAGS);
    }
#pragma unroll
    for (int g = 0; g < NGROUP; ++g) {
#pragma unroll
      for (int j = 0; j < IPW; ++j) {
        const int row = dma_row(g, j);
        const int phys = dma_phys(j);
        uint32_t offk, offv;
        if constexpr (GATHER) {
          const int idx = gidx[g * IPW + j];
          offk = idx >= 0 ? (uint32_t)idx * ROW + 16 * (phys ^ swz_k<CPR>(row)) : 0x80000000u;
          offv = idx >= 0 ? (uint32_t)idx * ROW + 16 * (phys ^ swz_v<CPR>(row)) : 0x80000000u;
        } else {
          offk = (uint32_t)row * ROW + 16 * (phys ^ swz_k<CPR>(row));
          offv = (uint32_t)row * ROW + 16 * (phys ^ swz_v<CPR>(row));
        }
        const int lds_off = (wave * IPW + j) * 1024;
        // dense: each split's K/V is read by its own workgroups only, once
        // (non-temporal); gathered pool rows are shared between tokens
        constexpr int CPOL = GATHER ? 0 : CPOL_NT;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rk, (__attribute__((address_space(3))) void*)(kgrp(g) + lds_off), 16, offk, 0, 0, CPOL);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rv, (__attribute__((address_space(3))) void*)(vgrp(g) + lds_off), 16, offv, 0, 0, CPOL);
      }
    }
  }
  if constexpr (GATHER) __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): sValid written

  const float c = p.scale_log2;
  const int jj = lane & 15;
  const int dsub = (lane >> 4) & 1;

  // Group g's keys are usable once this wave's DMAs up to group g have
  // landed (later groups may still be in flight) and a plain s_barrier has
  // published every wave's share.  (A __syncthreads() would add a release
  // fence, i.e. wait for all of them.)
  auto ready = [&](int g) __attribute__((always_inline)) {
    switch (g) {  // g is unrolled away; the wait needs an immediate count
      case 0: wait_vmcnt<2 * IPW * (NGROUP - 1)>(); break;
      case 1: wait_vmcnt<2 * IPW * (NGROUP - 2)>(); break;
      case 2: wait_vmcnt<2 * IPW * (NGROUP - 3)>(); break;
      default: wait_vmcnt<0>(); break;
    }
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  };
  // the K fragments of tile t (its group's LDS object, row-swizzled chunks)
  auto kfrag_of = [&](int t) __attribute__((always_inline)) {
    const int g = t / TPG;
    const int krow = (t % TPG) * KT + l32;
    const char* kr = kgrp(g) + krow * ROW;
    const int kx = swz_k<CPR>(g * GK + krow);
    return [=](int, int ds) __attribute__((always_inline)) {
      return *reinterpret_cast<const bf16x8*>(kr + 16 * ((2 * ds + hlf) ^ kx));
    };
  };
  // -inf for tile t's keys past the split or (gather) unusable
  auto mask_tile = [&](int t, f32x16 (&s)[1][NQB]) __attribute__((always_inline)) {
    const int kt0 = t * KT;
    bool any_masked = false;
    if constexpr (GATHER) any_masked = __any(lane < KT && !sValid[kt0 + (lane & (KT - 1))]);
    if (kt0 + KT > nk || (GATHER && any_masked)) {
      w.template mask<1>(s, hlf, [&](int kk) {
        const int key = kt0 + kk;
        if constexpr (GATHER) return key < nk && sValid[key] != 0;
        return key < nk;
      });
    }
  };

  // Software pipeline over the chunk's tiles: the QK^T MFMAs of tile t+1
  // carry tile t's exponentials (qk_next_softmax), then PV of tile t.  With
  // one wave per SIMD nothing else would overlap a tile's softmax.
  constexpr int MAXT = MAXK / KT;
  f32x16 s[1][NQB];
  if (n_tiles > 0) {
    ready(0);
    w.template qk<1>(s, kfrag_of(0));
    mask_tile(0, s);
  }
#pragma unroll
  for (int t = 0; t < MAXT; ++t) {
    if (t >= n_tiles) break;
    const bool has_next = t + 1 < n_tiles;
    if (has_next && (t + 1) % TPG == 0) ready((t + 1) / TPG);
    bf16x8 pf[NQB][NKS];
    float ls[NQB];
    f32x16 s_next[1][NQB];
    bool redo;
    if (has_next) {
      redo = w.qk_next_softmax(s_next, kfrag_of(t + 1), s, pf, c, ls);
    } else {
      redo = w.template softmax_fast<1>(s, pf, c, ls);
    }
    if (redo) w.template softmax_slow<1>(s, pf, c, ls);
    w.commit_l(ls);
    if (redo) w.rescale_o();
    if (has_next) mask_tile(t + 1, s_next);
    const int g = t / TPG;
    const int lt0 = (t % TPG) * KT;  // the tile's first row within its group's LDS object
    const char* sv = vgrp(g);
    w.template pv<NKS>(pf, [&](int ks, int db) {
      const int r0 = lt0 + 16 * ks + 4 * hlf + (jj >> 2);
      const int r1 = r0 + 8;
      const int ch = 4 * db + 2 * dsub + ((jj & 3) >> 1);
      const int sub = 8 * (jj & 1);
      return v_frag_tr(sv + r0 * ROW + 16 * (ch ^ swz_v<CPR>(g * GK + r0)) + sub,
                       sv + r1 * ROW + 16 * (ch ^ swz_v<CPR>(g * GK + r1)) + sub);
    });
    if (has_next) s[0][0] = s_next[0][0];
  }
  // Epilogue through LDS (the K/V groups are free once every wave is past
  // its last tile): wave w stages rows 0-15 in K group w, 16-31 in V group w.
  __syncthreads();
  char* const lo = kgrp(wave);
  char* const hi = vgrp(wave);
  constexpr int RB = HD * 4;  // room for fp32 rows; 16 rows fit a group
  static_assert(16 * RB <= GROUP_BYTES, "epilogue staging");
  w.store_lds(p, grow0, row0, split, lane,
              [&](int r) { return r < 16 ? lo + r * RB : hi + (r - 16) * RB; });
}

template <int HD, bool GATHER>
hipError_t launch_chunk_t(const FwdParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)p.tiles_per_group * p.n_groups * p.num_splits));
  hipLaunchKernelGGL((chunk_kernel<HD, GATHER>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

int chunk_max_keys(int hd) {
  switch (hd) {
    case 64: return ChunkShape<64>::MAXK;
    case 128: return ChunkShape<128>::MAXK;
    case 256: return ChunkShape<256>::MAXK;
    default: return 0;
  }
}

hipError_t launch_chunk(FwdParams p, int hd, hipStream_t stream) {
  constexpr int M_WG = 128;
  p.tiles_per_group = (p.rows_per_group + M_WG - 1) / M_WG;
  const bool gather = p.kv_idx != nullptr;
  switch (hd) {
    case 64:
      return gather ? launch_chunk_t<64, true>(p, stream) : launch_chunk_t<64, false>(p, stream);
    case 128:
      return gather ? launch_chunk_t<128, true>(p, stream) : launch_chunk_t<128, false>(p, stream);
    case 256:
      return gather ? launch_chunk_t<256, true>(p, stream) : launch_chunk_t<256, false>(p, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace fmha
