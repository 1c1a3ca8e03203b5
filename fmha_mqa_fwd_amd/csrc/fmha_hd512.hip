// Multi-query attention forward at head dim 512 for gfx950: the top-k row
// gather, and dense keys (decode splits, a sliding window).
//
// The shape is DeepSeek-V4's (page "May 24, 2026 — Session Start Plan", Key
// Numbers and File Map: head dim 512, Flash 64 query heads over top_k 512
// gathered keys, Pro 128 heads over top_k 1024): every query head of a token
// attends to the same s_k pool rows, picked by kv_idx (dsv4/kernels/cuda
// commit log, KV row gather); dense, every row of a batch attends to its
// s_k keys.
//
// Work split, as in the streaming kernel's head-dim-512 form: four waves = two
// blocks of 32 query rows x two halves of the head dim.  A wave holds its half
// of Q^T and of O^T, computes S^T over its 256 columns, and the two partials
// of a row block are summed through LDS before the (identical) softmax; each
// wave then does PV for its half of O.
//
// K/V movement (what this kernel changes):
//   * One LDS-DMA instruction moves one whole 1 KiB row.  M0 points at the
//     row's padded LDS slot and lane l takes bytes 16l..16l+15, so a lane's
//     offset is the row's pool offset + 16l, and the K and V instructions of a
//     row share it.  The padding (K +16 bytes, V +64 bytes per row) keeps the
//     operand reads free of bank conflicts with immediate offsets.
//   * The split's row offsets are staged in LDS once: gather, the index list
//     validated into pool byte offsets (in pool-region order when it has
//     ORDER_MIN_TILES tiles or more: then the workgroups running at one time
//     read rows from the same part of the pool and share L2 lines); dense,
//     the keys' offsets in the batch's K/V.  OOB marks an invalid entry or a
//     key past the split (the row reads as zeros and its logit is masked).  A
//     per-tile "has a masked key" bit lives in scalar registers.
//   * Two K and two V stages.  K(t+2) is issued as soon as every wave is past
//     QK^T(t) (the barrier of the S exchange), V(t+1) at the start of tile t;
//     each tile ends with a wait that leaves K(t+2) in flight.  The DMA is
//     issued from inline assembly, so the compiler adds no waits of its own.
//   * Gathered splits of 256 keys or more in launches of at least 512
//     workgroups run fwd512_pair_kernel instead: one K and one V stage, so two
//     workgroups share a CU and each computes while the other waits for its
//     rows (the same arithmetic in the same order, so the same results).
#include "fmha_device.h"

namespace fmha {
namespace {

using namespace dev;

constexpr int G5_HD = 512;
constexpr int G5_MAX_KEYS = 1024;  // a split's row offsets held in LDS

// One workgroup's work: `p` describes its key source, wc its row tile, group
// and split within that source; its partial (partial modes) goes to plane
// `plane`.  gather: the source is a pool read through kv_idx (a constant in
// the one-source kernels, per workgroup in the several-source one).
// NT: the K/V DMA is non-temporal (a dense split's keys are read once; in
// the several-source kernel, where the source decides at run time, plain).
// KPV: K(t+2) goes out between the PV MFMAs (measured faster for the gathered
// Flash top-k, slower for decode's short splits, which keep it right after
// the S exchange).
template <bool NT, bool KPV>
__device__ __forceinline__ void fwd512_body(const FwdParams& p, const bool gather,
                                            const WgCoords wc, const int plane) {
  constexpr int HD = G5_HD, HDW = HD / 2, QW = 32, KT = 32, WAVES = 4, NKS = KT / 16;
  constexpr int M_WG = 2 * QW;              // two row blocks
  constexpr int ROW = HD * 2;               // bytes per K/V row
  constexpr int KS = ROW + 16;              // padded LDS row strides
  constexpr int VS = ROW + 64;
  constexpr int RPW = KT / WAVES;           // rows each wave moves per tile and tensor
  static_assert(ROW == 64 * 16, "one DMA instruction per row");

  __shared__ __attribute__((aligned(16))) char sK0[KT * KS], sK1[KT * KS];
  __shared__ __attribute__((aligned(16))) char sV0[KT * VS], sV1[KT * VS];
  __shared__ __attribute__((aligned(16))) float sX[WAVES * 64 * 16];  // S^T partials
  __shared__ __attribute__((aligned(16))) uint32_t sOff[G5_MAX_KEYS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hlf = lane >> 5;
  const int dh = wave & 1;                  // which head-dim half this wave holds
  const int col0 = dh * HDW;

  const int tile = wc.tile, group = wc.group, split = wc.split;

  const int key_lo = split * p.chunk;
  const int key_hi = min(key_lo + p.chunk, p.s_k);
  const int nk = max(key_hi - key_lo, 0);  // <= G5_MAX_KEYS (host guarantees)
  const int n_tiles = (nk + KT - 1) / KT;
  const int row0 = tile * M_WG + (wave >> 1) * QW;
  const int64_t grow0 = (int64_t)group * p.rows_per_group;

  // gather: the pools; dense: this batch's keys (byte counts fit 32 bits: the
  // host checks rows * hd * 2)
  const int64_t kv0 = gather ? 0 : (int64_t)group * p.s_k * HD;
  const uint32_t kv_bytes = (uint32_t)(gather ? p.pool_rows : p.s_k) * ROW;
  const u32x4 rk = buffer_rsrc(p.k + kv0, kv_bytes);
  const u32x4 rv = buffer_rsrc(p.v + kv0, kv_bytes);
  const uint32_t lane16 = 16u * (uint32_t)lane;

  // the split's row offsets: gather, the index list validated into pool byte
  // offsets (ordered by pool region if long enough; sX is the sort's scratch
  // until the loop); dense, the keys' offsets in this batch's K/V.  The list entries
  // are loaded first and Q after them, so all of those loads are in flight
  // while the list is ordered.
  constexpr int SLOTS = G5_MAX_KEYS / 256;
  int idxv[SLOTS];
  if (gather) {
    const int32_t* ibase = p.kv_idx + (int64_t)group * p.s_k + key_lo;
#pragma unroll
    for (int e = 0; e < SLOTS; ++e) {
      const int i = tid + 256 * e;
      idxv[e] = i < nk ? ibase[i] : -1;
    }
  }
  Rows<HDW, QW, HD> w;
  w.load_q(p.q, grow0, row0, p.rows_per_group, l32, hlf, col0);
  if (gather && n_tiles >= ORDER_MIN_TILES) {
    const int sh = region_shift(p.pool_rows);
    uint32_t offv[SLOTS];
    int cls[SLOTS];
#pragma unroll
    for (int e = 0; e < SLOTS; ++e) {
      const bool ok = idxv[e] >= 0 && idxv[e] < p.pool_rows;
      offv[e] = ok ? (uint32_t)idxv[e] * ROW : OOB;
      cls[e] = ok ? idxv[e] >> sh : REGION_NONE;
    }
    order_by_region<WAVES, SLOTS>(offv, cls, n_tiles * KT, sOff, reinterpret_cast<int*>(sX),
                                  wave, lane);
  } else if (gather) {
#pragma unroll
    for (int e = 0; e < SLOTS; ++e) {
      const int i = tid + 256 * e;
      if (i < n_tiles * KT)
        sOff[i] = (idxv[e] >= 0 && idxv[e] < p.pool_rows) ? (uint32_t)idxv[e] * ROW : OOB;
    }
  } else {
    for (int i = tid; i < n_tiles * KT; i += 256)
      sOff[i] = i < nk ? (uint32_t)(key_lo + i) * ROW : OOB;
  }
  // Q and the list are in before any DMA is issued, so the compiler's own
  // waits for them stay out of the loop
  wait_vmcnt<0>();
  __syncthreads();

  uint64_t tile_masked = 0;  // bit t: tile t has a masked key
  for (int r = 0; r < n_tiles; r += 2) {  // each wave reads the list two tiles at a time
    const int i = r * KT + lane;
    const uint64_t b = __ballot(i < n_tiles * KT && sOff[min(i, G5_MAX_KEYS - 1)] == OOB);
    tile_masked |= (((uint32_t)b != 0) ? 1ull : 0ull) << r;
    tile_masked |= (((uint32_t)(b >> 32) != 0) ? 1ull : 0ull) << (r + 1);
  }

  // this lane's DMA offsets for the RPW rows this wave moves in tile t
  // (rows RPW*wave .. +RPW-1); past the last tile every row reads as zeros
  struct Offs {
    uint32_t o[RPW];
  };
  auto offsets = [&](int t) __attribute__((always_inline)) {
    Offs r;
    if (t < n_tiles) {
      const u32x4* src = reinterpret_cast<const u32x4*>(sOff + t * KT + wave * RPW);
#pragma unroll
      for (int h = 0; h < RPW / 4; ++h) {
        const u32x4 x = src[h];
#pragma unroll
        for (int e = 0; e < 4; ++e) r.o[4 * h + e] = x[e] + lane16;
      }
    } else {
#pragma unroll
      for (int j = 0; j < RPW; ++j) r.o[j] = OOB;
    }
    return r;
  };
  auto issue_row = [&](const u32x4& rsrc, const Offs& o, char* buf, int stride, int j)
      __attribute__((always_inline)) {
    if constexpr (NT)
      dma16_nt(rsrc, (uint32_t)(uintptr_t)(buf + (wave * RPW + j) * stride), o.o[j]);
    else
      dma16(rsrc, (uint32_t)(uintptr_t)(buf + (wave * RPW + j) * stride), o.o[j]);
  };
  auto issue = [&](const u32x4& rsrc, const Offs& o, char* buf, int stride)
      __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < RPW; ++j) issue_row(rsrc, o, buf, stride, j);
  };
  auto barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS accesses are done
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  };

  const float c = p.scale_log2;
  const int jj = lane & 15;
  const int dsub = (lane >> 4) & 1;
  // per-lane operand offsets within a stage (see fwd_kernel): K row l32,
  // bytes 16*hlf of each 32-byte step; V rows/columns of the transposed read
  const int k_lane = l32 * KS + 16 * hlf + 2 * col0;
  const int v_lane = (4 * hlf + (jj >> 2)) * VS + 2 * (16 * dsub + 4 * (jj & 3)) + 2 * col0;
  f32x4* const x_mine = reinterpret_cast<f32x4*>(sX + (wave * 64 + lane) * 16);
  const f32x4* const x_theirs = reinterpret_cast<const f32x4*>(sX + ((wave ^ 1) * 64 + lane) * 16);

  Offs next;  // offsets of tile t+1 (its K is in flight, its V is issued at the start of t)
  auto step = [&](int t, char* kcur, const char* vcur, char* vnext)
      __attribute__((always_inline)) {
    // V(t+1), one row after each of the first RPW QK^T MFMAs (the DMA issue
    // then overlaps the matrix unit)
    f32x16 s[1][1];
    w.qk_mid(s, [&](int, int ds) __attribute__((always_inline)) {
      return *reinterpret_cast<const bf16x8*>(kcur + k_lane + ds * 32);
    }, [&](int ds) __attribute__((always_inline)) {
      if (ds < RPW) issue_row(rv, next, vnext, VS, ds);
    });
    // S^T = this wave's partial + its partner's (same lanes, same layout)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      x_mine[i] = f32x4{s[0][0][4 * i], s[0][0][4 * i + 1], s[0][0][4 * i + 2], s[0][0][4 * i + 3]};
    barrier();  // every wave is past QK^T(t): K(t)'s stage is free
    const Offs ahead = offsets(t + 2);
    if constexpr (!KPV) issue(rk, ahead, kcur, KS);  // K(t+2)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 o = x_theirs[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) s[0][0][4 * i + e] += o[e];
    }
    if ((tile_masked >> t) & 1) {
      const int kbase = t * KT;
      w.template mask<1>(s, hlf, [&](int kk) { return sOff[kbase + kk] != OOB; });
    }
    bf16x8 pf[1][NKS];
    if (w.template softmax<1>(s, pf, c)) w.rescale_o();
    w.template pv_mid<NKS>(pf, [&](int ks, int db) __attribute__((always_inline)) {
      const char* a = vcur + v_lane + 16 * ks * VS + 64 * db;
      return v_frag_tr(a, a + 8 * VS);
    }, [&](int i) __attribute__((always_inline)) {
      if constexpr (KPV) {
        if (i < RPW) issue_row(rk, ahead, kcur, KS, i);  // K(t+2)
      }
    });
    next = ahead;
    // K(t+1) and V(t+1) have landed; K(t+2) may still be in flight
    wait_vmcnt<RPW>();
    barrier();
  };

  if (n_tiles > 0) {
    const Offs o0 = offsets(0);
    issue(rk, o0, sK0, KS);
    issue(rv, o0, sV0, VS);
    next = offsets(1);
    issue(rk, next, sK1, KS);
    wait_vmcnt<RPW>();  // K(0) and V(0) have landed
    barrier();
    for (int t = 0; t < n_tiles; t += 2) {
      step(t, sK0, sV0, sV1);
      if (t + 1 < n_tiles) step(t + 1, sK1, sV1, sV0);
    }
  }
  // every DMA (also the zero-filling ones past the end) has landed and every
  // wave is past its reads before the K stages are reused for the epilogue
  wait_vmcnt<0>();
  barrier();
  constexpr int RB_BF16 = HDW * 2;
  static_assert(2 * QW * RB_BF16 <= KT * KS, "epilogue staging");
  if (is_bf16(p.out_mode)) {
    char* const region = ((wave >> 1) == 0 ? sK0 : sK1) + dh * QW * RB_BF16;
    w.store_lds(p, grow0, row0, plane, lane, [&](int r) { return region + r * RB_BF16; }, col0,
                dh == 0);
    return;
  }
  w.store(p, grow0, row0, plane, l32, hlf, col0, dh == 0);
}

// Long gathered splits, two workgroups per CU: one K and one V stage (72 KiB of
// LDS), the S exchange in the K stage once every wave is past QK^T, K(t+1)
// issued after the exchange and V(t+1) after PV(t); a tile waits for its K
// before QK^T and for its V only after the exchange.  A workgroup waits for
// each tile; the other workgroup on its CU computes meanwhile.
__device__ __forceinline__ void fwd512_pair_body(const FwdParams& p, const WgCoords wc,
                                                 const int plane) {
  constexpr int HD = G5_HD, HDW = HD / 2, QW = 32, KT = 32, WAVES = 4, NKS = KT / 16;
  constexpr int M_WG = 2 * QW;
  constexpr int ROW = HD * 2;
  constexpr int KS = ROW + 16;
  constexpr int VS = ROW + 64;
  constexpr int RPW = KT / WAVES;
  static_assert(ROW == 64 * 16, "one DMA instruction per row");
  static_assert(WAVES * 64 * 16 * 4 <= KT * KS, "S exchange in the K stage");

  __shared__ __attribute__((aligned(16))) char sK[KT * KS];
  __shared__ __attribute__((aligned(16))) char sV[KT * VS];
  __shared__ __attribute__((aligned(16))) uint32_t sOff[G5_MAX_KEYS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hlf = lane >> 5;
  const int dh = wave & 1;
  const int col0 = dh * HDW;
  const int tile = wc.tile, group = wc.group;
  const int key_lo = wc.split * p.chunk;
  const int key_hi = min(key_lo + p.chunk, p.s_k);
  const int nk = max(key_hi - key_lo, 0);
  const int n_tiles = (nk + KT - 1) / KT;
  const int row0 = tile * M_WG + (wave >> 1) * QW;
  const int64_t grow0 = (int64_t)group * p.rows_per_group;
  const u32x4 rk = buffer_rsrc(p.k, (uint32_t)p.pool_rows * ROW);
  const u32x4 rv = buffer_rsrc(p.v, (uint32_t)p.pool_rows * ROW);
  const uint32_t lane16 = 16u * (uint32_t)lane;

  // the list, validated and (ORDER_MIN_TILES tiles or more) in pool-region
  // order; sV is the sort's scratch before the first V DMA
  constexpr int SLOTS = G5_MAX_KEYS / 256;
  int idxv[SLOTS];
  {
    const int32_t* ibase = p.kv_idx + (int64_t)group * p.s_k + key_lo;
#pragma unroll
    for (int e = 0; e < SLOTS; ++e) {
      const int i = tid + 256 * e;
      idxv[e] = i < nk ? ibase[i] : -1;
    }
  }
  Rows<HDW, QW, HD> w;
  w.load_q(p.q, grow0, row0, p.rows_per_group, l32, hlf, col0);
  if (n_tiles >= ORDER_MIN_TILES) {
    const int sh = region_shift(p.pool_rows);
    uint32_t offv[SLOTS];
    int cls[SLOTS];
#pragma unroll
    for (int e = 0; e < SLOTS; ++e) {
      const bool ok = idxv[e] >= 0 && idxv[e] < p.pool_rows;
      offv[e] = ok ? (uint32_t)idxv[e] * ROW : OOB;
      cls[e] = ok ? idxv[e] >> sh : REGION_NONE;
    }
    order_by_region<WAVES, SLOTS>(offv, cls, n_tiles * KT, sOff, reinterpret_cast<int*>(sV),
                                  wave, lane);
  } else {
#pragma unroll
    for (int e = 0; e < SLOTS; ++e) {
      const int i = tid + 256 * e;
      if (i < n_tiles * KT)
        sOff[i] = (idxv[e] >= 0 && idxv[e] < p.pool_rows) ? (uint32_t)idxv[e] * ROW : OOB;
    }
  }
  wait_vmcnt<0>();
  __syncthreads();
  uint64_t tile_masked = 0;
  for (int r = 0; r < n_tiles; r += 2) {
    const int i = r * KT + lane;
    const uint64_t b = __ballot(i < n_tiles * KT && sOff[min(i, G5_MAX_KEYS - 1)] == OOB);
    tile_masked |= (((uint32_t)b != 0) ? 1ull : 0ull) << r;
    tile_masked |= (((uint32_t)(b >> 32) != 0) ? 1ull : 0ull) << (r + 1);
  }
  // the scratch (sV) and the list are read before any DMA lands in sV
  __syncthreads();

  auto issue = [&](const u32x4& rsrc, int t, char* buf, int stride) __attribute__((always_inline)) {
    uint32_t o[RPW];
    if (t < n_tiles) {
      const u32x4* src = reinterpret_cast<const u32x4*>(sOff + t * KT + wave * RPW);
#pragma unroll
      for (int h = 0; h < RPW / 4; ++h) {
        const u32x4 x = src[h];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[4 * h + e] = x[e] + lane16;
      }
    } else {
#pragma unroll
      for (int j = 0; j < RPW; ++j) o[j] = OOB;
    }
#pragma unroll
    for (int j = 0; j < RPW; ++j)
      dma16(rsrc, (uint32_t)(uintptr_t)(buf + (wave * RPW + j) * stride), o[j]);
  };
  auto barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  };
  const float c = p.scale_log2;
  const int jj = lane & 15;
  const int dsub = (lane >> 4) & 1;
  const int k_lane = l32 * KS + 16 * hlf + 2 * col0;
  const int v_lane = (4 * hlf + (jj >> 2)) * VS + 2 * (16 * dsub + 4 * (jj & 3)) + 2 * col0;
  float* const sX = reinterpret_cast<float*>(sK);
  f32x4* const x_mine = reinterpret_cast<f32x4*>(sX + (wave * 64 + lane) * 16);
  const f32x4* const x_theirs = reinterpret_cast<const f32x4*>(sX + ((wave ^ 1) * 64 + lane) * 16);

  if (n_tiles > 0) {
    issue(rk, 0, sK, KS);
    issue(rv, 0, sV, VS);
  }
  for (int t = 0; t < n_tiles; ++t) {
    wait_vmcnt<RPW>();
    barrier();  // K(t) has landed; V(t), issued after it, may still be in flight
    f32x16 s[1][1];
    w.template qk<1>(s, [&](int, int ds) __attribute__((always_inline)) {
      return *reinterpret_cast<const bf16x8*>(sK + k_lane + ds * 32);
    });
    barrier();  // every wave is past QK^T(t): the K stage holds the exchange
#pragma unroll
    for (int i = 0; i < 4; ++i)
      x_mine[i] = f32x4{s[0][0][4 * i], s[0][0][4 * i + 1], s[0][0][4 * i + 2], s[0][0][4 * i + 3]};
    barrier();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 o = x_theirs[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) s[0][0][4 * i + e] += o[e];
    }
    wait_vmcnt<0>();
    barrier();  // V(t) has landed, and every partial is read: K(t+1) may land
    issue(rk, t + 1, sK, KS);
    if ((tile_masked >> t) & 1) {
      const int kbase = t * KT;
      w.template mask<1>(s, hlf, [&](int kk) { return sOff[kbase + kk] != OOB; });
    }
    bf16x8 pf[1][NKS];
    if (w.template softmax<1>(s, pf, c)) w.rescale_o();
    w.template pv<NKS>(pf, [&](int ks, int db) __attribute__((always_inline)) {
      const char* a = sV + v_lane + 16 * ks * VS + 64 * db;
      return v_frag_tr(a, a + 8 * VS);
    });
    barrier();  // every wave is past PV(t): V(t+1) may land
    issue(rv, t + 1, sV, VS);
  }
  wait_vmcnt<0>();
  barrier();
  constexpr int RB_BF16 = HDW * 2;
  static_assert(2 * QW * RB_BF16 <= KT * KS, "epilogue staging");
  if (is_bf16(p.out_mode)) {
    char* const region = ((wave >> 1) == 0 ? sK : sV) + dh * QW * RB_BF16;
    w.store_lds(p, grow0, row0, plane, lane, [&](int r) { return region + r * RB_BF16; }, col0,
                dh == 0);
    return;
  }
  w.store(p, grow0, row0, plane, l32, hlf, col0, dh == 0);
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd512_pair_kernel(FwdParams p) {
  const WgCoords wc =
      wg_coords(blockIdx.x, p.tiles_per_group, p.n_groups, p.n_groups * p.num_splits);
  fwd512_pair_body(p, wc, wc.split);
}

template <bool GATHER>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fwd512_kernel(FwdParams p) {
  const WgCoords wc =
      wg_coords(blockIdx.x, p.tiles_per_group, p.n_groups, p.n_groups * p.num_splits);
  fwd512_body<!GATHER, GATHER>(p, GATHER, wc, wc.split);  // gathered pool rows are shared
}

// Several key sources in one launch: workgroup blockIdx.x belongs to the last
// source whose first workgroup is at or before it, and is placed within that
// source exactly as a one-source launch would place it.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fwd512_sources_kernel(SourcesParams sp) {
  const int bid = blockIdx.x;
  SourceParams src = sp.src[0];
#pragma unroll
  for (int i = 1; i < MAX_SOURCES; ++i)
    if (i < sp.n_src && bid >= sp.src[i].wg_begin) src = sp.src[i];
  FwdParams p = sp.base;
  p.k = src.k;
  p.v = src.v;
  p.kv_idx = src.kv_idx;
  p.s_k = src.s_k;
  p.pool_rows = src.pool_rows;
  p.chunk = src.chunk;
  p.num_splits = src.num_splits;
  p.n_groups = src.n_groups;
  p.rows_per_group = src.rows_per_group;
  p.tiles_per_group = src.tiles_per_group;
  const WgCoords wc = wg_coords(bid - src.wg_begin, src.tiles_per_group, src.n_groups,
                                src.n_groups * src.num_splits);
  fwd512_body<false, false>(p, src.kv_idx != nullptr, wc, src.plane_begin + wc.split);
}

}  // namespace

int fwd512_max_keys() { return G5_MAX_KEYS; }

hipError_t launch_fwd512(const FwdParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)p.tiles_per_group * p.n_groups * p.num_splits));
  // long gathered splits and enough workgroups for two per CU (256 CUs):
  // the single-stage kernel, two per CU; otherwise the double-buffered one
  if (p.kv_idx != nullptr && p.chunk >= 256 && grid.x >= 512)
    hipLaunchKernelGGL(fwd512_pair_kernel, grid, dim3(256), 0, stream, p);
  else if (p.kv_idx != nullptr)
    hipLaunchKernelGGL(fwd512_kernel<true>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(fwd512_kernel<false>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_fwd512_sources(SourcesParams sp, hipStream_t stream) {
  if (sp.n_src < 1 || sp.n_src > MAX_SOURCES) return hipErrorInvalidValue;
  int64_t wg = 0;
  for (int i = 0; i < sp.n_src; ++i) {
    SourceParams& s = sp.src[i];
    if (s.chunk > G5_MAX_KEYS) return hipErrorInvalidValue;
    s.tiles_per_group = (s.rows_per_group + 63) / 64;  // 64-row tiles
    s.wg_begin = (int)wg;
    wg += (int64_t)s.tiles_per_group * s.n_groups * s.num_splits;
  }
  if (wg < 1 || wg > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fwd512_sources_kernel, dim3((unsigned)wg), dim3(256), 0, stream, sp);
  return hipGetLastError();
}

}  // namespace fmha
