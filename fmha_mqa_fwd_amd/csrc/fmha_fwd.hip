// Multi-query attention forward for gfx950 (MI355X, CDNA4): streaming kernel.
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
//   * head dims 64/128/256 ("D1 Status Summary");
//   * optional row gather of the s_k = top_k selected keys from a KV pool (same
//     page "Key Numbers"; dsv4/kernels/cuda commit log, KV row gather).
//
// How it is mapped onto CDNA4 (our design, not the pages' Blackwell one):
//   * Head-packed M: the rows of a group (all (t, h) of a batch, or all heads of
//     a token) share K/V, so a workgroup takes WAVES*QW consecutive rows and
//     every K/V tile staged in LDS serves all of them.
//   * S^T = K . Q^T and O^T = V^T . P^T with v_mfma_f32_32x32x16_bf16, P kept in
//     registers, the online softmax in-lane (fmha_device.h).
//   * K/V tiles are moved global -> LDS by LDS-DMA buffer loads
//     (buffer_load_dwordx4 ... lds): no staging registers, no VALU, and keys
//     past the end of the split (or out-of-range pool rows) read as zeros from
//     beyond the buffer descriptor.  A DMA instruction fills 1 KiB of LDS
//     contiguously; rows are padded (K by 16 bytes for the ds_read_b128 operand
//     reads, V by 64 bytes for the ds_read_b64_tr_b16 reads, both free of bank
//     conflicts) and the lanes that land on pad bytes read out-of-range zeros,
//     so every operand read is a per-lane base plus an immediate offset.
//   * Double buffering: tile t+1 is DMA'd while tile t is computed; each buffer
//     is its own LDS object and the loop is unrolled by two.  Dense tiles are
//     DMA'd from inline assembly, one instruction after each QK^T MFMA, and
//     waited for explicitly before the tile's barrier; gathered tiles use the
//     compiler-tracked builtin, whose waits the compiler keeps per buffer.
//     One barrier per tile.
//   * Several workgroups share a CU where registers allow, so one wave's
//     softmax overlaps other waves' MFMAs.
#include <type_traits>

#include "fmha_device.h"

namespace fmha {
namespace {

using namespace dev;

// Padded LDS row strides (bytes): K rows are read as ds_read_b128 by 16 lanes
// at 16 consecutive rows and one column (16-byte pad: 16 distinct bank
// groups); V rows by ds_read_b64_tr_b16, whose 32-lane halves read 4
// consecutive rows x 64 bytes (64-byte pad: 4 disjoint bank ranges).
template <int HD>
struct Lds {
  static constexpr int ROW = HD * 2;
  static constexpr int K_STRIDE = ROW + 16;
  static constexpr int V_STRIDE = ROW + 64;
};


// Head dims above 256: DSPLIT = 2 waves share the same QW rows, each holding
// half of the head dim (its Q^T columns, its O^T rows): each computes a
// partial S over its half, the two partials are summed through LDS (the
// softmax needs the whole contraction first), both run the same softmax and
// each does PV for its half.
template <int HD>
struct DSplit {
  static constexpr int value = HD > 256 ? 2 : 1;
};

template <int HD, int QW, int KT, int WAVES, bool GATHER, int WPE>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void fwd_kernel(FwdParams p) {
  constexpr int THREADS = WAVES * 64;
  constexpr int NQB = QW / 32;
  constexpr int NKB = KT / 32;   // 32-key row blocks of S^T per tile
  constexpr int NKS = KT / 16;   // 16-key contraction steps of PV per tile
  constexpr int DSPLIT = DSplit<HD>::value;
  constexpr int HDW = HD / DSPLIT;  // head-dim columns one wave holds
  constexpr int M_WG = WAVES / DSPLIT * QW;
  static_assert(DSPLIT == 1 || (NQB == 1 && NKB == 1), "split head dim: one S block per wave");
  constexpr int ROW = Lds<HD>::ROW;
  constexpr int KS = Lds<HD>::K_STRIDE;
  constexpr int VS = Lds<HD>::V_STRIDE;
  constexpr int NKI = (KT * KS + 1023) / 1024;   // DMA instructions per K tile
  constexpr int NVI = (KT * VS + 1023) / 1024;   // ... per V tile
  constexpr int KJ = (NKI + WAVES - 1) / WAVES;  // per wave (upper bound)
  constexpr int VJ = (NVI + WAVES - 1) / WAVES;
  static_assert(QW % 32 == 0 && KT % 32 == 0 && HD % 32 == 0, "tile shape");
  static_assert(KT <= THREADS, "one index per thread");

  __shared__ __attribute__((aligned(1024))) char sK0[NKI * 1024], sK1[NKI * 1024];
  __shared__ __attribute__((aligned(1024))) char sV0[NVI * 1024], sV1[NVI * 1024];
  __shared__ int sIdx[GATHER ? 3 : 1][KT];    // gather: pool rows of a tile (-1 = masked)
  __shared__ int sValid[GATHER ? 2 : 1][KT];  // gather: key usable, per K buffer
  // split head dim: each wave's partial S^T (16 floats per lane)
  __shared__ __attribute__((aligned(16))) float sX[DSPLIT > 1 ? WAVES * 64 * 16 : 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // scalar (DMA guards and M0 in scalar code) where it measured faster: not
  // with the head dim split over waves, whose register pressure it raises
  const int wave = DSPLIT == 1 ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;
  const int l32 = lane & 31;
  const int hlf = lane >> 5;

  const WgCoords wc =
      wg_coords(blockIdx.x, p.tiles_per_group, p.n_groups, p.n_groups * p.num_splits);
  const int tile = wc.tile, group = wc.group, split = wc.split;

  const int key_lo = split * p.chunk;
  const int key_hi = min(key_lo + p.chunk, p.s_k);
  const int n_tiles = key_hi > key_lo ? (key_hi - key_lo + KT - 1) / KT : 0;
  const int dh = wave % DSPLIT;              // which head-dim part this wave holds
  const int col0 = dh * HDW;
  const int row0 = tile * M_WG + wave / DSPLIT * QW;  // first row of this wave in its group
  const int64_t grow0 = (int64_t)group * p.rows_per_group;
  const uint16_t* kbase = GATHER ? p.k : p.k + (int64_t)group * p.s_k * HD;
  const uint16_t* vbase = GATHER ? p.v : p.v + (int64_t)group * p.s_k * HD;
  const int32_t* ibase = GATHER ? p.kv_idx + (int64_t)group * p.s_k : nullptr;

  // ---- per-lane DMA geometry (same for every tile): instruction j of this
  // wave fills LDS bytes [1024*(wave + WAVES*j), +1024) of a tile buffer; lane
  // `lane` of it lands in row r = pos/STRIDE at column byte c = pos%STRIDE.
  // kr/vr: that row (-1: pad bytes or past the tile); kc/vc: the column.
  int kr[KJ], kc[KJ], vr[VJ], vc[VJ];
#pragma unroll
  for (int j = 0; j < KJ; ++j) {
    const int inst = wave + WAVES * j;
    const int pos = inst * 1024 + lane * 16;
    const int r = pos / KS, cc = pos % KS;
    const bool ok = inst < NKI && cc < ROW && r < KT;
    kr[j] = ok ? r : -1;
    kc[j] = cc;
  }
#pragma unroll
  for (int j = 0; j < VJ; ++j) {
    const int inst = wave + WAVES * j;
    const int pos = inst * 1024 + lane * 16;
    const int r = pos / VS, cc = pos % VS;
    const bool ok = inst < NVI && cc < ROW && r < KT;
    vr[j] = ok ? r : -1;
    vc[j] = cc;
  }

  // Gather: thread j < KT fetches the pool row of key j of tile t.
  auto fetch_idx = [&](int t) __attribute__((always_inline)) {
    const int key = key_lo + t * KT + tid;
    int idx = -1;
    if (tid < KT && t < n_tiles && key < key_hi) idx = ibase[key];
    return (idx >= 0 && idx < p.pool_rows) ? idx : -1;
  };

  // Dense keys: the DMA is issued from inline assembly (the compiler tracks
  // none of it, so it can sit between the MFMAs of QK^T without costing
  // registers), and every wait for it is explicit.  The descriptors of tile t
  // cover keys t0 .. key_hi-1: later rows read as zeros.
  auto dense_rsrc = [&](int t, u32x4& rk4, u32x4& rv4) __attribute__((always_inline)) {
    const int t0 = key_lo + t * KT;
    const uint32_t nbytes = (uint32_t)((key_hi - t0) * ROW);
    rk4 = buffer_rsrc(kbase + (int64_t)t0 * HD, nbytes);
    rv4 = buffer_rsrc(vbase + (int64_t)t0 * HD, nbytes);
  };
  // slot q of this wave's dense DMA of a tile: K instruction j = q (q < KJ), else V j = q - KJ
  auto dense_slot = [&](int q, const u32x4& rk4, const u32x4& rv4, char* kbuf, char* vbuf)
      __attribute__((always_inline)) {
    const bool isk = q < KJ;
    const int j = isk ? q : q - KJ;
    const int inst = wave + WAVES * j;
    if (inst < (isk ? NKI : NVI)) {
      const int r = isk ? kr[j] : vr[j];
      const uint32_t off = r >= 0 ? (uint32_t)r * ROW + (uint32_t)(isk ? kc[j] : vc[j]) : OOB;
      dma16(isk ? rk4 : rv4, (uint32_t)(uintptr_t)((isk ? kbuf : vbuf) + inst * 1024), off);
    }
  };
  // DMA of tile t into (kbuf, vbuf); gather rows come from sIdx[ib].
  auto issue = [&](int t, char* kbuf, char* vbuf, int ib) __attribute__((always_inline)) {
    if constexpr (!GATHER) {
      u32x4 rk4, rv4;
      dense_rsrc(t, rk4, rv4);
#pragma unroll
      for (int q = 0; q < KJ + VJ; ++q) dense_slot(q, rk4, rv4, kbuf, vbuf);
      return;
    }
    __amdgpu_buffer_rsrc_t rk, rv;
    rk = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, p.pool_rows * ROW, BUF_FLAGS);
    rv = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, p.pool_rows * ROW, BUF_FLAGS);
#pragma unroll
    for (int j = 0; j < KJ; ++j) {
      const int inst = wave + WAVES * j;
      if (inst < NKI) {
        uint32_t off = OOB;
        if (kr[j] >= 0) {
          const int idx = sIdx[ib][kr[j]];
          off = idx >= 0 ? (uint32_t)idx * ROW + kc[j] : OOB;
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rk, (__attribute__((address_space(3))) void*)(kbuf + inst * 1024), 16, off, 0, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < VJ; ++j) {
      const int inst = wave + WAVES * j;
      if (inst < NVI) {
        uint32_t off = OOB;
        if (vr[j] >= 0) {
          const int idx = sIdx[ib][vr[j]];
          off = idx >= 0 ? (uint32_t)idx * ROW + vc[j] : OOB;
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rv, (__attribute__((address_space(3))) void*)(vbuf + inst * 1024), 16, off, 0, 0, 0);
      }
    }
  };

  Rows<HDW, QW, HD> w;
  w.load_q(p.q, grow0, row0, p.rows_per_group, l32, hlf, col0);
  const float c = p.scale_log2;

  // Per-lane LDS byte offsets of the MFMA operands within a tile buffer.
  //  K (A of S^T, ds_read_b128): row 32*kb + l32, bytes 32*ds + 16*hlf.
  //  V (A of O^T, ds_read_b64_tr_b16): lane (jj, dsub, hlf) of K-step ks,
  //  d block db and half r reads row 16*ks + 8*r + 4*hlf + jj/4, columns
  //  32*db + 16*dsub + 4*(jj%4) .. +3; the 16-lane transpose then hands lane
  //  (d = 32*db + lane%32, hlf) the keys 16*ks + 8*(e/4) + 4*hlf + e%4, e = 0..7,
  //  which is where S^T's accumulator layout put that lane's P values.
  const int jj = lane & 15;
  const int dsub = (lane >> 4) & 1;
  const int k_lane = l32 * KS + 16 * hlf + 2 * col0;
  const int v_lane = (4 * hlf + (jj >> 2)) * VS + 2 * (16 * dsub + 4 * (jj & 3)) + 2 * col0;

  // One tile: compute tile t from (kcur, vcur) while tile t+1 streams into
  // (knext, vnext).  Buffers are distinct LDS objects in each unrolled copy.
  auto step = [&](int t, const char* kcur, const char* vcur, char* knext, char* vnext, int vb)
      __attribute__((always_inline)) {
    const int t0 = key_lo + t * KT;
    const bool have_next = t + 1 < n_tiles;
    int idx_ahead = -1;
    // dense one-block tiles: the DMA of tile t+1 goes out one instruction
    // after each QK^T MFMA (its issue then overlaps the matrix unit; ~1%
    // faster per prefill call than issuing it all before QK^T)
    constexpr bool MID = !GATHER && NKB == 1 && NQB == 1 && DSPLIT == 1;
    if (have_next) {
      if constexpr (GATHER) {
        // validity of tile t+1 for its K buffer, then its DMA
        if (tid < KT) sValid[vb ^ 1][tid] = sIdx[(t + 1) % 3][tid] >= 0;
        issue(t + 1, knext, vnext, (t + 1) % 3);
        idx_ahead = fetch_idx(t + 2);  // written to LDS after the compute
      } else if constexpr (!MID) {
        issue(t + 1, knext, vnext, 0);
      }
    }

    f32x16 s[NKB][NQB];
    auto kfrag = [&](int kb, int ds) __attribute__((always_inline)) {
      return *reinterpret_cast<const bf16x8*>(kcur + k_lane + kb * 32 * KS + ds * 32);
    };
    if constexpr (MID) {
      constexpr int NDS_ = HDW / 16;
      u32x4 rk4, rv4;
      dense_rsrc(t + 1, rk4, rv4);
      w.qk_mid(s, kfrag, [&](int ds) __attribute__((always_inline)) {
        if (ds < KJ + VJ && have_next) dense_slot(ds, rk4, rv4, knext, vnext);
      });
      if (have_next) {
#pragma unroll
        for (int q = NDS_; q < KJ + VJ; ++q) dense_slot(q, rk4, rv4, knext, vnext);
      }
    } else {
      w.template qk<NKB>(s, kfrag);
    }
    if constexpr (DSPLIT == 2) {
      // S^T = this wave's partial + its partner's (same lanes, same layout)
      f32x4* mine = reinterpret_cast<f32x4*>(sX + (wave * 64 + lane) * 16);
      const f32x4* theirs = reinterpret_cast<const f32x4*>(sX + ((wave ^ 1) * 64 + lane) * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        mine[i] = f32x4{s[0][0][4 * i], s[0][0][4 * i + 1], s[0][0][4 * i + 2], s[0][0][4 * i + 3]};
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the partial is in LDS
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 o = theirs[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) s[0][0][4 * i + e] += o[e];
      }
    }
    bool masked = !GATHER && (t0 + KT > key_hi);
    if constexpr (GATHER) masked = __any(lane < KT && !sValid[vb][lane & (KT - 1)]);
    if (masked) {
      w.template mask<NKB>(s, hlf, [&](int kk) {
        return GATHER ? (sValid[vb][kk] != 0) : (t0 + kk < key_hi);
      });
    }
    bf16x8 pf[NQB][NKS];
    if (w.template softmax<NKB>(s, pf, c)) w.rescale_o();
    w.template pv<NKS>(pf, [&](int ks, int db) {
      const char* a = vcur + v_lane + 16 * ks * VS + 64 * db;
      return v_frag_tr(a, a + 8 * VS);
    });

    if constexpr (GATHER) {
      if (have_next && tid < KT) sIdx[(t + 2) % 3][tid] = idx_ahead;
    }
    // tile t+1 has landed (dense: the explicit wait; gather: this barrier's
    // release fence waits for every compiler-tracked DMA) and no wave reads
    // (kcur, vcur) any more
    if constexpr (!GATHER) wait_vmcnt<0>();
    __syncthreads();
  };

  if (n_tiles > 0) {
    if constexpr (GATHER) {
      const int i0 = fetch_idx(0);
      const int i1 = fetch_idx(1);
      if (tid < KT) {
        sIdx[0][tid] = i0;
        sIdx[1][tid] = i1;
        sValid[0][tid] = i0 >= 0;
      }
      __syncthreads();
    }
    issue(0, sK0, sV0, 0);
    if constexpr (!GATHER) wait_vmcnt<0>();  // tile 0 has landed
    if constexpr (GATHER) {
      const int i2 = fetch_idx(2);
      if (tid < KT) sIdx[2][tid] = i2;
    }
    __syncthreads();
  }
  for (int t = 0; t < n_tiles; t += 2) {
    step(t, sK0, sV0, sK1, sV1, 0);
    if (t + 1 < n_tiles) step(t + 1, sK1, sV1, sK0, sV0, 1);
  }

  // Epilogue through LDS for bf16 outputs: each wave stages its 32 rows in a
  // tile buffer of its own (sK0, sK1, sV0, sV1), so that memory sees whole
  // 16-byte-per-lane row segments; otherwise each lane stores its own pieces.
  // The last barrier of the loop has retired every read of those buffers.
  constexpr int RB_BF16 = HDW * 2;
  static_assert(QW == 32, "epilogue staging assumes 32 rows per wave");
  if constexpr (WAVES == 4 && QW * RB_BF16 <= NKI * 1024) {
    if (is_bf16(p.out_mode)) {
      char* const region = wave == 0 ? sK0 : wave == 1 ? sK1 : wave == 2 ? sV0 : sV1;
      w.store_lds(p, grow0, row0, split, lane, [&](int r) { return region + r * RB_BF16; }, col0,
                  dh == 0);
      return;
    }
  }
  w.store(p, grow0, row0, split, l32, hlf, col0, dh == 0);
}

// ------------------------------------------------------------------------
// Gather kernel for splits of at most GSW_MAX_KEYS keys (hd 64/128/256).
// Same tile shape, padded LDS rows and operand reads as fwd_kernel; what
// differs is how the gathered rows are moved:
//   * the split's index list is validated once and staged in LDS as pool
//     byte offsets (OOB for an invalid entry or a key past the split), and a
//     per-tile "has a masked key" bit is kept in scalar registers, so the
//     loop issues no global loads and tests no index per key;
//   * the list is staged in pool-region order (order_by_region): the result
//     does not depend on the order of the keys, and the workgroups running at
//     one time then read rows from the same part of the pool;
//   * the per-lane DMA offsets of tile t+1 are read from that list one tile
//     ahead (during tile t-1), so no DMA waits on an LDS read;
//   * every wave issues the same number of DMA instructions per tile (slots
//     past a tile's last instruction write zeros to a spare KiB of LDS), and
//     the DMA is issued from inline assembly with one explicit vmcnt wait per
//     tile, so the compiler adds no waits of its own.
// Without a swizzle the operand addresses are a base register plus immediate
// offsets, which keeps the hd 128 kernel within 168 VGPRs: three workgroups
// per CU.
constexpr int GSW_MAX_KEYS = 1024;  // a split's index list held in LDS

template <int HD, int WPE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void fwd_gather_staged_kernel(FwdParams p) {
  constexpr int WAVES = 4, QW = 32, KT = 32, NKB = 1, NKS = KT / 16;
  constexpr int M_WG = WAVES * QW;
  constexpr int ROW = Lds<HD>::ROW;
  constexpr int KS = Lds<HD>::K_STRIDE;
  constexpr int VS = Lds<HD>::V_STRIDE;
  constexpr int NKI = (KT * KS + 1023) / 1024;   // DMA instructions per K tile
  constexpr int NVI = (KT * VS + 1023) / 1024;   // ... per V tile
  constexpr int KJ = (NKI + WAVES - 1) / WAVES;  // per wave (slots past NKI: the spare KiB)
  constexpr int VJ = (NVI + WAVES - 1) / WAVES;

  __shared__ __attribute__((aligned(1024))) char sK0[NKI * 1024], sK1[NKI * 1024];
  __shared__ __attribute__((aligned(1024))) char sV0[NVI * 1024], sV1[NVI * 1024];
  __shared__ __attribute__((aligned(1024))) char sSpare[1024];
  __shared__ uint32_t sOff[GSW_MAX_KEYS + KT];  // the list, then a tile of OOB

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hlf = lane >> 5;

  const WgCoords wc =
      wg_coords(blockIdx.x, p.tiles_per_group, p.n_groups, p.n_groups * p.num_splits);
  const int tile = wc.tile, group = wc.group, split = wc.split;

  const int key_lo = split * p.chunk;
  const int key_hi = min(key_lo + p.chunk, p.s_k);
  const int nk = max(key_hi - key_lo, 0);  // <= GSW_MAX_KEYS (host guarantees)
  const int n_tiles = (nk + KT - 1) / KT;
  const int row0 = tile * M_WG + wave * QW;
  const int64_t grow0 = (int64_t)group * p.rows_per_group;
  const int32_t* ibase = p.kv_idx + (int64_t)group * p.s_k + key_lo;

  // DMA geometry (as fwd_kernel): slot j of this wave is instruction
  // wave + 4j, whose lane `lane` fills tile bytes [1024 inst + 16 lane, +16):
  // row r (-1: pad bytes, past the tile, or a spare slot) and column byte c
  int kr[KJ], vr[VJ];
  uint32_t kc[KJ], vc[VJ];
#pragma unroll
  for (int j = 0; j < KJ; ++j) {
    const int inst = wave + WAVES * j;
    const int pos = inst * 1024 + lane * 16;
    const int r = pos / KS, cc = pos % KS;
    kr[j] = (inst < NKI && cc < ROW && r < KT) ? r : -1;
    kc[j] = kr[j] >= 0 ? (uint32_t)cc : 0xFFFFFFFFu;  // a pad lane's offset saturates past any pool
  }
#pragma unroll
  for (int j = 0; j < VJ; ++j) {
    const int inst = wave + WAVES * j;
    const int pos = inst * 1024 + lane * 16;
    const int r = pos / VS, cc = pos % VS;
    vr[j] = (inst < NVI && cc < ROW && r < KT) ? r : -1;
    vc[j] = vr[j] >= 0 ? (uint32_t)cc : 0xFFFFFFFFu;
  }
  const u32x4 rk = buffer_rsrc(p.k, (uint32_t)p.pool_rows * ROW);
  const u32x4 rv = buffer_rsrc(p.v, (uint32_t)p.pool_rows * ROW);
  struct Offs {
    uint32_t k[KJ], v[VJ];
  };
  // the list entries of this lane's rows of tile t, read unconditionally (a
  // tile past the last reads the OOB tile after the list, a pad slot row 0,
  // whose value its column then pushes out of range) so that the reads carry
  // no branch and no wait of their own; the compiler waits for them where
  // issue uses them, a tile later
  auto offsets = [&](int t) __attribute__((always_inline)) {
    Offs o;
    const int base = min(t, n_tiles) * KT;
#pragma unroll
    for (int j = 0; j < KJ; ++j) o.k[j] = sOff[base + max(kr[j], 0)];
#pragma unroll
    for (int j = 0; j < VJ; ++j) o.v[j] = sOff[base + max(vr[j], 0)];
    return o;
  };
  // slot q of a tile's DMA from its list entries: K instruction q (q < KJ),
  // else V instruction q - KJ.  Entry + column in one saturating add: a
  // usable row's offset plus its column stays inside the pool; OOB (2^31,
  // beyond any pool's byte count) plus a column, or anything plus a pad
  // lane's all-ones column, lands past the pool and reads zeros.
  auto issue_slot = [&](const Offs& o, int q, char* kbuf, char* vbuf)
      __attribute__((always_inline)) {
    if (q < KJ) {
      const int inst = wave + WAVES * q;
      const uint32_t off = __builtin_elementwise_add_sat(o.k[q], kc[q]);
      dma16(rk, (uint32_t)(uintptr_t)(inst < NKI ? kbuf + inst * 1024 : sSpare), off);
    } else {
      const int j = q - KJ;
      const int inst = wave + WAVES * j;
      const uint32_t off = __builtin_elementwise_add_sat(o.v[j], vc[j]);
      dma16(rv, (uint32_t)(uintptr_t)(inst < NVI ? vbuf + inst * 1024 : sSpare), off);
    }
  };
  auto issue = [&](const Offs& o, char* kbuf, char* vbuf) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < KJ + VJ; ++q) issue_slot(o, q, kbuf, vbuf);
  };
  auto barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS accesses are done
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  };

  Rows<HD, QW> w;
  const float c = p.scale_log2;
  const int jj = lane & 15;
  const int dsub = (lane >> 4) & 1;
  // per-lane operand offsets within a tile buffer (see fwd_kernel)
  const int k_lane = l32 * KS + 16 * hlf;
  const int v_lane = (4 * hlf + (jj >> 2)) * VS + 2 * (16 * dsub + 4 * (jj & 3));
  Offs ahead;                // offsets of tile t+1, read during tile t-1
  uint64_t tile_masked = 0;  // bit t: tile t has a masked key

  constexpr int NDS = HD / 16;
  auto step = [&](int t, const char* kcur, const char* vcur, char* knext, char* vnext)
      __attribute__((always_inline)) {
    // tile t+1's DMA, one instruction after each QK^T MFMA (its issue then
    // overlaps the matrix unit), from the entries read a tile ago
    f32x16 s[NKB][1];
    w.qk_mid(s, [&](int, int ds) __attribute__((always_inline)) {
      return *reinterpret_cast<const bf16x8*>(kcur + k_lane + ds * 32);
    }, [&](int ds) __attribute__((always_inline)) {
      if (ds < KJ + VJ) issue_slot(ahead, ds, knext, vnext);
    });
#pragma unroll
    for (int q = NDS; q < KJ + VJ; ++q) issue_slot(ahead, q, knext, vnext);
    ahead = offsets(t + 2);  // read under this tile's softmax and PV
    if ((tile_masked >> t) & 1) {
      const int kbase = t * KT;
      w.template mask<NKB>(s, hlf, [&](int kk) { return sOff[kbase + kk] != OOB; });
    }
    bf16x8 pf[1][NKS];
    if (w.template softmax<NKB>(s, pf, c)) w.rescale_o();
    w.template pv<NKS>(pf, [&](int ks, int db) {
      const char* a = vcur + v_lane + 16 * ks * VS + 64 * db;
      return v_frag_tr(a, a + 8 * VS);
    });
    wait_vmcnt<0>();  // tile t+1 has landed
    barrier();
  };

  // the split's index list, validated, as pool byte offsets in pool-region
  // order (sV1 is the sort's scratch until tile 1 is DMA'd; the splits that
  // reach this kernel have more keys than the whole-chunk kernel takes, 5
  // tiles or more).  Every entry of this thread is loaded before any is used,
  // and Q after them, so all of those loads are in flight together.
  constexpr int IPT = GSW_MAX_KEYS / 256;  // list entries per thread
  int idxv[IPT];
#pragma unroll
  for (int e = 0; e < IPT; ++e) {
    const int i = tid + 256 * e;
    idxv[e] = i < nk ? ibase[i] : -1;
  }
  w.load_q(p.q, grow0, row0, p.rows_per_group, l32, hlf);
  static_assert(NVI * 1024 >= GSW_MAX_KEYS / 64 * 64 * 4, "sort scratch");
  const int n_list = n_tiles * KT;
  const int sh = region_shift(p.pool_rows);
  uint32_t offv[IPT];
  int cls[IPT];
#pragma unroll
  for (int e = 0; e < IPT; ++e) {
    const bool ok = idxv[e] >= 0 && idxv[e] < p.pool_rows;
    offv[e] = ok ? (uint32_t)idxv[e] * ROW : OOB;
    cls[e] = ok ? idxv[e] >> sh : REGION_NONE;
  }
  const int n_usable = order_by_region<WAVES, IPT>(offv, cls, n_list, sOff,
                                                   reinterpret_cast<int*>(sV1), wave, lane);
  // the entries that read nothing are last: tiles n_usable / KT .. n_tiles - 1
  // have a masked key (n_tiles <= 32)
  if (n_usable < n_list)
    tile_masked = ((1ull << n_tiles) - 1) & ~((1ull << (n_usable / KT)) - 1);
  if (tid < KT) sOff[n_list + tid] = OOB;  // what tiles past the last read
  // Q and the list are in before any DMA is issued, so the compiler's own
  // waits for them stay out of the loop
  wait_vmcnt<0>();
  __syncthreads();
  if (n_tiles > 0) {
    issue(offsets(0), sK0, sV0);
    ahead = offsets(1);
    wait_vmcnt<0>();  // tile 0 has landed
    barrier();
    for (int t = 0; t < n_tiles; t += 2) {
      step(t, sK0, sV0, sK1, sV1);
      if (t + 1 < n_tiles) step(t + 1, sK1, sV1, sK0, sV0);
    }
  }
  // every wave is past its reads before the buffers are reused for the epilogue
  wait_vmcnt<0>();
  barrier();
  constexpr int RB_BF16 = HD * 2;
  if constexpr (QW * RB_BF16 <= NKI * 1024) {
    if (is_bf16(p.out_mode)) {
      char* const region = wave == 0 ? sK0 : wave == 1 ? sK1 : wave == 2 ? sV0 : sV1;
      w.store_lds(p, grow0, row0, split, lane, [&](int r) { return region + r * RB_BF16; });
      return;
    }
  }
  w.store(p, grow0, row0, split, l32, hlf);
}

template <int HD, int WPE>
hipError_t launch_gather_staged(const FwdParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)p.tiles_per_group * p.n_groups * p.num_splits));
  hipLaunchKernelGGL((fwd_gather_staged_kernel<HD, WPE>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

struct Shape {
  int qw, kt, waves, wpe;
  int rows() const { return waves * qw; }  // rows per workgroup (before a head-dim split)
};

// Rows per workgroup of each kernel (fwd_kernel for dense keys and for
// gather splits of more than GSW_MAX_KEYS keys, fwd_gather_staged_kernel
// otherwise): 4 waves x 32 rows, or 2 row blocks of 32 at hd 512.  32 rows per
// wave keeps a wave within 170 registers (dense hd <= 128 and the staged
// gather at hd 128: three waves per SIMD) or 256 (the long-split gather form,
// 64-key tiles: two waves per SIMD), so one wave's softmax overlaps other
// waves' MFMAs.  hd 256 needs the whole register file: one wave per SIMD.
Shape pick_shape(int hd, bool gather) {
  if (hd > 256) return {32, 32, 2, 1};  // 2 row blocks x 2 head-dim halves = 4 waves
  if (hd >= 256) return {32, 32, 4, 1};
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

// a split whose keys fit in LDS whole goes to the whole-chunk kernel
bool use_chunk(const FwdParams& p, int hd) {
  const int mk = chunk_max_keys(hd);
  return mk > 0 && p.chunk <= mk;
}

}  // namespace

int64_t fwd_grid_size(const FwdParams& p, int hd) {
  const Shape sh = pick_shape(hd, p.kv_idx != nullptr);
  const int64_t m_wg = use_chunk(p, hd) ? 128 : (int64_t)sh.rows();
  const int64_t tiles = (p.rows_per_group + m_wg - 1) / m_wg;
  return tiles * p.n_groups * p.num_splits;
}

hipError_t launch_fwd(FwdParams p, int hd, hipStream_t stream) {
  // a split that fits in LDS whole is staged at once (decode shapes)
  if (use_chunk(p, hd)) return launch_chunk(p, hd, stream);
  const bool gather = p.kv_idx != nullptr;
  const Shape sh = pick_shape(hd, gather);
  const int m_wg = sh.rows();
  p.tiles_per_group = (p.rows_per_group + m_wg - 1) / m_wg;
  switch (hd) {
    case 64:
      return gather ? (p.chunk <= GSW_MAX_KEYS ? launch_gather_staged<64, 4>(p, stream)
                                               : launch_t<64, 32, 64, 4, 2, true>(p, stream))
                    : launch_t<64, 32, 32, 4, 3, false>(p, stream);
    case 128:
      return gather ? (p.chunk <= GSW_MAX_KEYS ? launch_gather_staged<128, 3>(p, stream)
                                               : launch_t<128, 32, 64, 4, 2, true>(p, stream))
                    : launch_t<128, 32, 32, 4, 3, false>(p, stream);
    case 256:
      return gather ? (p.chunk <= GSW_MAX_KEYS ? launch_gather_staged<256, 1>(p, stream)
                                               : launch_t<256, 32, 32, 4, 1, true>(p, stream))
                    : launch_t<256, 32, 32, 4, 1, false>(p, stream);
    case 512:
      if (p.chunk <= fwd512_max_keys()) return launch_fwd512(p, stream);
      return gather ? launch_t<512, 32, 32, 4, 1, true>(p, stream)
                    : launch_t<512, 32, 32, 4, 1, false>(p, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace fmha
