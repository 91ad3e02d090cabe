// Forward KPage attention for gfx950 (MI355X, CDNA4).
//
// KPage paper, section 3.2: every work item is one query block of one
// (batch, head).  Its K/V page walk (8 Page16 regions per step for M128 x N128,
// 16 for M64 x N256) is consumed in tiles of 4 pages (64 key rows).  Each page is
// a contiguous 16-row run of the original K/V tensors and is copied straight from
// global memory into LDS with 16-byte direct-to-LDS loads (section 3.2.3); no
// compacted copy exists in HBM.  The consumer is a flash-attention step on the
// assembled tile: bf16 MFMA for Q K^T and P V with fp32 accumulation, and a softmax
// over the walk (section 3.2.4: invalid rows are set to -inf before the row maximum,
// and only on tiles at or past the end of the fully valid prefix) whose maximum is
// fixed by the first sub-tile, with an exact re-run for the rare item that needs a
// running maximum (below).
//
// Work split.  A workgroup has 4 waves and two workgroups share a CU, so every
// SIMD runs two waves of different items that drift apart: one wave's vector
// work issues while the other's matrix work runs.  Each wave copies one K and one
// V page of every tile, owns 32 query rows of the item and a fixed key range of
// every tile, walked as sub-tiles of 32 keys.  Route M128 x N128 (section 3.2.2):
// 4 query groups, every wave takes all 64 keys of a tile (2 sub-tiles).  Route
// M64 x N256: 2 query groups x 2 key halves, 1 sub-tile per wave per tile.  Each
// wave keeps its own running maximum, sum and output; waves that share query
// rows are merged once at the end.  A group item (up to four query blocks of at most
// 32 rows over the union of their walks) runs on the M128 route with one member per
// wave.  One launch covers both routes, in the launch order of the plan's order table
// (per head its M128 items, then its M64 items).
//
// Matrix layout per wave (v_mfma_f32_32x32x16_bf16, 32 cycles each):
//   S^T (key x query) = K . Q^T : A = K rows from LDS, B = Q rows kept in VGPRs.
//     A lane then holds 16 keys of one query column, so the row maximum is a
//     lane-local reduction plus one exchange with lane ^ 32.
//   O^T (dim x query) = V^T . P^T : B = the probabilities straight from the S^T
//     accumulators (same lane layout), A = V read transposed from LDS with
//     ds_read_b64_tr_b16.  The output column of a lane is again its own query,
//     so the per-query rescaling needs no cross-lane traffic.
//
// Software pipeline.  Sub-tile i is processed in three parts that run in
// different sub-iterations: its scores S_i = K_i Q^T (MFMA), its softmax (VALU)
// and its product P_i V_i (MFMA).  Sub-iteration i issues the MFMAs of S_{i+1}
// and of P_{i-1} V_{i-1} and, between them, the softmax of S_i.
//
// Running maximum.  In the fast kernel a query's maximum is fixed by the first
// sub-tile that has a valid key for it and never moves again: probabilities are
// exp2(s - m) with a stale m, so the output accumulators are never rescaled
// inside the loop (which keeps them in the matrix-core registers).  This is
// exact as long as later scores exceed m by less than 2^64 (no overflow of P,
// O or l in fp32); an item where some score rises further is marked in its first
// LSE row and recomputed by the second kernel, which raises the maximum whenever a
// sub-tile exceeds it by more than 2^8 and rescales O and l then.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device.hpp"
#include "kpage.h"
#include "tile_common.hpp"

namespace kpage {
namespace {

// 4 waves per workgroup, two workgroups per CU; the walk is consumed in 4-page tiles
// (64 keys), one K and one V page per wave.
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTilePages = 4;
constexpr float kLimit = 64.0f;  // fast kernel: largest rise of a score over the fixed maximum (base 2)
constexpr float kRaise = 8.0f;   // exact kernel: raise the maximum only past this margin (base 2)
// First LSE row of an item the fast kernel leaves to the exact kernel: a quiet NaN no
// real result produces (LSE is finite or -inf).
constexpr uint32_t kRedoMark = 0x7FC0DA0Au;
constexpr int kExactBlocks = 512;  // exact re-run grid cap: 2 workgroups per CU

// Page of wave j in tile t of a walk (one scalar load).
__device__ __forceinline__ int32_t fwd_page(c_i32 *walk, int t, int j) { return walk[kTilePages * t + j]; }

// MASK values of a sub-iteration: no masking, a runtime check, or masking always.
constexpr int kMaskNone = 0, kMaskCheck = 1, kMaskAlways = 2;

// LDS of one workgroup, the same for both routes: K tiles 0/1, then V tiles 0/1 (at the
// end the per-wave partial outputs), and the per-wave row statistics of the merge.
template <int D>
struct FwdLds {
  __attribute__((aligned(1024))) char tiles[4 * 16 * kTilePages * D * 2];
  float stat_m[kWaves][32];
  float stat_l[kWaves][32];
  int redo_any;
};

// One work item of route ROUTE: `item` indexes the route's item array.
template <int D, int ROUTE, bool EXACT>
__device__ __forceinline__ void fwd_item(const FwdArgs &args, int item, FwdLds<D> &lds) {
  constexpr int CH = D / 8;          // 16-byte chunks per row
  constexpr int DS = D / 16;         // MFMA k-steps over the head dimension
  constexpr int ND = D / 32;         // 32-wide output blocks over the head dimension
  constexpr int M = ROUTE;           // query rows of the work item
  constexpr int NQG = M / 32;        // query groups of 32 rows
  constexpr int NKG = kWaves / NQG;  // key groups per tile
  constexpr int KW = 16 * kTilePages / NKG;  // keys of a tile per wave
  constexpr int NH = KW / 32;        // 32-key sub-tiles per wave per tile
  constexpr int TILE_BYTES = 16 * kTilePages * D * 2;
  constexpr int LOADS = 16 * CH / 64;  // direct loads per wave per tile and tensor

  static_assert(sizeof(FwdLds<D>::tiles) == 4 * TILE_BYTES, "two K and two V tiles");
  char *smem = lds.tiles;
  float(&stat_m)[kWaves][32] = lds.stat_m;
  float(&stat_l)[kWaves][32] = lds.stat_l;
  int &redo_any = lds.redo_any;

  char *kbuf0 = smem, *kbuf1 = smem + TILE_BYTES, *vbuf0 = smem + 2 * TILE_BYTES, *vbuf1 = smem + 3 * TILE_BYTES;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int g = lane >> 5;           // lane half: selects 8 of the 16 k values of an MFMA operand
  const int l32 = lane & 31;

  const FwdItem it = args.items[item];
  const int bh = it.bh;
  // 4-page tiles up to the last one holding a real page; the all-dummy tiles of the
  // walk's step padding are neither copied nor computed
  const int n_tiles = (it.n_pages + kTilePages - 1) / kTilePages;
  const int n_sub = n_tiles * NH;
  const int full_tiles = it.n_full / kTilePages;  // tiles inside the fully valid prefix
  const int qg = wave % NQG;
  const int keyoff = (wave / NQG) * KW;  // first key of this wave in a tile
  // this wave's query rows (a group item's wave holds the rows of its own member block)
  const WaveRows wr = wave_rows(it, args.groups, qg);
  // a query group without valid rows computes nothing: the wave still copies its pages
  // and meets every barrier (none sits inside the compute below), and its rows are
  // written as O = 0, LSE = -inf like every row past c_q
  const bool idle = wr.rows <= 0;

  const char *kh = (const char *)args.k + (int64_t)bh * args.seq_kv * D * 2;
  const char *vh = (const char *)args.v + (int64_t)bh * args.seq_kv * D * 2;
  c_i32 *walk = (c_i32 *)(args.pages + it.walk_off);
  c_u32 *vwords = (c_u32 *)(args.valid + wr.valid_off);

  // Q rows of this wave as MFMA B operands: qreg[s] = Q[q0 + l32][16s + 8g .. +8]
  bf16x8 qreg[DS];
  {
    const int q0 = 128 * wr.block + wr.row0;
    const bf16x8 *qh = (const bf16x8 *)((const char *)args.q + ((int64_t)bh * args.seq_q + q0) * D * 2);
    const bool ok = l32 < wr.rows;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      bf16x8 x = qh[l32 * (D / 8) + 2 * s + g];
      if (!ok) x = bf16x8{};
      qreg[s] = x;
    }
  }
  if (n_tiles > 0) load_page<D, kSwzRow>(kh, fwd_page(walk, 0, wave), (lds_char *)kbuf0, 16 * wave, lane);
  if (n_tiles > 1) load_page<D, kSwzRow>(kh, fwd_page(walk, 1, wave), (lds_char *)kbuf1, 16 * wave, lane);
  if (ROUTE == 128 && n_tiles > 0) load_page<D, kSwzTr>(vh, fwd_page(walk, 0, wave), (lds_char *)vbuf0, 16 * wave, lane);

  f32x16 oacc[ND];
#pragma unroll
  for (int n = 0; n < ND; ++n) oacc[n] = f32x16{};
  float m2 = kNegInf;    // running maximum of the scaled scores (base-2 units)
  float l_run = 0.f;     // this lane's part of the running sum
  bool over = false;     // fast kernel: a score rose past the fixed maximum + kLimit
  const float c2 = args.scale_log2;

  // lane-constant parts of the LDS addresses
  const int k_row_off = (keyoff + l32) * D * 2;
  const int k_swz = lane & (CH - 1);
  const int sl = lane & 15;
  const int mgrp = lane >> 4;
  const int v_row_off = (keyoff + 4 * g + (sl >> 2)) * D * 2;
  const int v_chunk_lane = 2 * (mgrp & 1) + ((sl & 3) >> 1);
  const int v_swz = vswz(sl >> 2) & (CH - 1);
  const int v_byte = (sl & 1) * 8;

  // Scores and probabilities ping-pong between two register sets selected by the
  // parity of the sub-tile index (a compile-time value at every call site).
  f32x16 sacc[2];       // [parity]: scores of the sub-tile in softmax / of the next one
  bf16x8 pacc[2][2];    // [parity][hh]: probabilities of a sub-tile

  auto read_v_op = [&](const lds_char *vrow) __attribute__((always_inline)) -> bf16x8 {
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)vrow);
    const s16x4 hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(vrow + 8 * D * 2));
    const bf16x4 lo_b = __builtin_bit_cast(bf16x4, lo), hi_b = __builtin_bit_cast(bf16x4, hi);
    return bf16x8{lo_b[0], lo_b[1], lo_b[2], lo_b[3], hi_b[0], hi_b[1], hi_b[2], hi_b[3]};
  };
  // S^T of one sub-tile (32 keys x 32 queries) from the K tile in `kt`
  auto qk = [&](const lds_char *kt, int half, f32x16 &acc) __attribute__((always_inline)) {
    acc = f32x16{};
    if (idle) return;
    const lds_char *base = kt + k_row_off + half * 32 * D * 2;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      const bf16x8 kop = *(const __attribute__((address_space(3))) bf16x8 *)(base + (((2 * s + g) ^ k_swz) * 16));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qreg[s], acc, 0, 0, 0);
    }
  };
  // O^T += V^T P^T for one sub-tile from the V tile in `vt`
  auto pv = [&](const lds_char *vt, int half, const bf16x8 *p) __attribute__((always_inline)) {
    if (idle) return;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const lds_char *vrow = vt + v_row_off + (32 * half + 16 * hh) * D * 2;
#pragma unroll
      for (int n = 0; n < ND; ++n) {
        const bf16x8 vop = read_v_op(vrow + ((4 * n + v_chunk_lane) ^ v_swz) * 16 + v_byte);
        oacc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, p[hh], oacc[n], 0, 0, 0);
      }
    }
  };
  // validity word of sub-tile `sub` for this wave's keys (its 32 keys, 16 bits per page)
  auto sub_word = [&](int sub) __attribute__((always_inline)) -> uint32_t {
    return vwords[(sub / NH) * (kTilePages / 2) + (keyoff >> 5) + sub % NH];
  };
  // exact masking of invalid key rows of sub-tile `sub` (its 32 keys = one validity word)
  auto mask = [&](int sub, f32x16 &sc) __attribute__((always_inline)) {
    const uint32_t word = sub_word(sub);
    // register r holds key acc_row(r, g): its bit is wave-uniform in each lane half, so
    // the condition is a scalar lane mask and each score costs one select
    const float ninf = kNegInf;
    static_for<16>([&](auto r_c) __attribute__((always_inline)) {
      constexpr int R = decltype(r_c)::value;
      sc[R] = select_lanes(row_lane_mask<R>(word), sc[R], ninf);
    });
  };
  float alpha = 1.f;  // exact kernel: rescale factor owed by the last softmax
  float nm_fix = 0.f;  // fast kernel: -(fixed maximum) once the first sub-tile set it
  bool pending = false;
  // softmax of sc into p_out (the sequential form: exact kernel and peeled sub-iterations)
  auto softmax = [&](const f32x16 &sc, bf16x8 *p_out) __attribute__((always_inline)) {
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; r += 2) mx = max3(mx, sc[r], sc[r + 1]);
    mx = half_max(mx) * c2;
    if (EXACT) {
      const bool up = mx > m2 + kRaise;
      const float mnew = up ? mx : m2;
      alpha = up ? __builtin_amdgcn_exp2f(m2 - mnew) : 1.f;
      m2 = mnew;
      pending = __builtin_amdgcn_ballot_w64(up) != 0;
    } else {
      // the first sub-tile with a valid key fixes the maximum; sums taken before it (in
      // the loop's sub-iterations, against 0) would not match it: the item is re-run
      const bool first = m2 == kNegInf;
      over = over || (!first && mx > m2 + kLimit) || (first && l_run != 0.f);
      m2 = first ? mx : m2;
    }
    const float nm = m2 == kNegInf ? 0.f : -m2;
    float rs = 0.f;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[8 * hh + e], c2, nm));
        rs += p;
        p_out[hh][e] = (__bf16)p;
      }
    l_run = EXACT ? l_run * alpha + rs : l_run + rs;
  };
  auto rescale = [&]() __attribute__((always_inline)) {
    if (EXACT && pending) {
#pragma unroll
      for (int n = 0; n < ND; ++n) oacc[n] *= alpha;
      pending = false;
    }
  };

  // Full sub-iteration of the fast kernel, hand-interleaved: the DS MFMAs of S_{i+1}
  // and the 2 ND MFMAs of P_{i-1} V_{i-1} alternate one per chunk, and the softmax
  // of S_i is cut into slices placed between them.  A scheduling fence closes every
  // second chunk, so the order written here is the order issued.  K and V operands
  // are read from LDS two products ahead of their MFMAs.
  auto fused = [&](auto par, const lds_char *kb, int khalf, const lds_char *vb, int vhalf, auto probs_only)
                   __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    // probabilities of S_i only: S_{i+1} and P_{i-1} are known to hold no key of this wave
    constexpr bool ONLY_P = decltype(probs_only)::value;
    constexpr int VOPS = 2 * ND, NM = DS + VOPS;
    constexpr int SLICES = 4;  // probabilities of 4 scores each
    static_assert(DS == VOPS, "QK and PV products alternate one to one");
    const f32x16 &sc = sacc[P];
    f32x16 &sn = sacc[1 - P];
    bf16x8 *po = pacc[P];
    const bf16x8 *pp = pacc[1 - P];
    bf16x8 kop[DS], vop[VOPS];
    const lds_char *kbase = kb + k_row_off + khalf * 32 * D * 2;
    const lds_char *vbase = vb + v_row_off + vhalf * 32 * D * 2;
    auto read_k = [&](auto s_c) __attribute__((always_inline)) {
      constexpr int S = decltype(s_c)::value;
      kop[S] = *(const __attribute__((address_space(3))) bf16x8 *)(kbase + (((2 * S + g) ^ k_swz) * 16));
    };
    auto read_v = [&](auto j_c) __attribute__((always_inline)) {
      constexpr int J = decltype(j_c)::value, HH = J / ND, N = J % ND;
      vop[J] = read_v_op(vbase + 16 * HH * D * 2 + ((4 * N + v_chunk_lane) ^ v_swz) * 16 + v_byte);
    };
    float rs0 = 0.f, rs1 = 0.f;
    // slice k: probabilities of scores 4 k .. 4 k + 3 (exp2, two partial row sums,
    // bf16 packs) against the maximum fixed by the first sub-tile (nm_fix = -m2); no
    // per-sub-tile maximum: a rise past the fixed maximum shows in the row sum, which
    // the epilogue checks
    auto slice = [&](auto k_c) __attribute__((always_inline)) {
      constexpr int K = decltype(k_c)::value;
      {
        constexpr int R = 4 * K;
        const float nm = nm_fix;
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] = __builtin_fmaf(sc[R + e], c2, nm);
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] = __builtin_amdgcn_exp2f(p[e]);
        rs0 += p[0];
        rs1 += p[1];
        rs0 += p[2];
        rs1 += p[3];
#pragma unroll
        for (int e = 0; e < 4; ++e) po[R / 8][R % 8 + e] = (__bf16)p[e];
      }
    };
    if constexpr (ONLY_P) {
      static_for<SLICES>([&](auto k_c) __attribute__((always_inline)) { slice(k_c); });
      l_run += rs0 + rs1;
      sn = f32x16{};  // S_{i+1}: every key masked by the next sub-iteration
      return;
    }
    read_k(ic<0>{});
    read_k(ic<1>{});
    read_v(ic<0>{});
    read_v(ic<1>{});
    __builtin_amdgcn_sched_barrier(0);
    static_for<NM>([&](auto c_c) __attribute__((always_inline)) {
      constexpr int C = decltype(c_c)::value, KK = C / 2;
      if constexpr (C % 2 == 0) {
        if constexpr (KK + 2 < DS) read_k(ic<KK + 2>{});
        sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[KK], qreg[KK], KK == 0 ? f32x16{} : sn, 0, 0, 0);
      } else {
        constexpr int HH = KK / ND, N = KK % ND;
        if constexpr (KK + 2 < VOPS) read_v(ic<KK + 2>{});
        oacc[N] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[KK], pp[HH], oacc[N], 0, 0, 0);
      }
      static_for<SLICES>([&](auto k_c) __attribute__((always_inline)) {
        constexpr int K = decltype(k_c)::value;
        if constexpr (K * NM / SLICES == C) slice(ic<K>{});
      });
      if constexpr (C % 2 == 1) __builtin_amdgcn_sched_barrier(0);
    });
    l_run += rs0 + rs1;
  };

  // Sub-iteration i: S_{i+1} (if HAS_QK), softmax of S_i, P_{i-1} V_{i-1} (if HAS_PV).
  // PAR = i & 1.  KB / VB: LDS tiles holding the keys of sub-tile i+1 and the values of
  // sub-tile i-1.  In the exact kernel the rescale owed by sub-tile i-1 runs first,
  // after P_{i-2} V_{i-2} and before P_{i-1} V_{i-1}.
  auto step = [&](auto has_qk, auto has_pv, auto par, auto masking, const lds_char *kb, const lds_char *vb,
                  int i) __attribute__((always_inline)) {
    constexpr bool HAS_QK = decltype(has_qk)::value;
    constexpr bool HAS_PV = decltype(has_pv)::value;
    constexpr int P = decltype(par)::value;
    constexpr int MASK = decltype(masking)::value;
    if (idle) return;
    rescale();
    if (MASK == kMaskAlways || (MASK == kMaskCheck && i / NH >= full_tiles)) mask(i, sacc[P]);
    __builtin_amdgcn_sched_barrier(0);
    if (!EXACT && HAS_QK && HAS_PV) {
      // Past the valid prefix a run of sub-tiles may hold no key of this wave (pages a
      // group member did not select, dummy pages): their probabilities are exactly 0.
      // When sub-tiles i - 1 and i + 1 both hold none, S_{i+1} (masked to -inf by the
      // next sub-iteration) and P_{i-1} V_{i-1} are skipped; the probabilities of S_i
      // are still taken.  M128 route only: with both variants the M64 loop spills.
      if (NH == 2 && MASK == kMaskAlways && sub_word(i + 1) == 0u && sub_word(i - 1) == 0u)
        fused(par, kb, (i + 1) % NH, vb, (i - 1 + NH) % NH, ic<1>{});
      else
        fused(par, kb, (i + 1) % NH, vb, (i - 1 + NH) % NH, ic<0>{});
    } else {
      if (HAS_QK) qk(kb, (i + 1) % NH, sacc[1 - P]);
      softmax(sacc[P], pacc[P]);
      if (HAS_PV) pv(vb, (i - 1 + NH) % NH, pacc[1 - P]);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  constexpr ic<1> T;
  constexpr ic<0> F;
  const lds_char *K0 = (const lds_char *)kbuf0, *K1 = (const lds_char *)kbuf1;
  const lds_char *V0 = (const lds_char *)vbuf0, *V1 = (const lds_char *)vbuf1;

  if (n_sub > 0) {
    // The steady-state loops run only full sub-iterations (scores of the next
    // sub-tile, softmax, product of the previous one).  The first and the last
    // sub-iterations are peeled, and sub-tiles that may need masking run in a loop
    // of their own, so no loop body carries a branch around its MFMA work.
    if (NH == 2) {
      // Sub-tile i = 2t + h lives in tile t.  Before sub-iteration 2t + 1: K_{t+1} and
      // V_t are resident; K_{t+2} and V_{t+1} are then issued into the buffers of K_t
      // and V_{t-1}, which no wave reads any more.
      if (n_tiles > 1) wait_vmcnt<2 * LOADS>(); else wait_vmcnt<LOADS>();
      barrier();
      qk(K0, 0, sacc[0]);
      step(T, F, ic<0>{}, ic<kMaskCheck>{}, K0, V0, 0);  // S_1 comes from the same tile
      nm_fix = m2 == kNegInf ? 0.f : -m2;
      // tile body t: sub-iterations 2t + 1 (softmax of tile t) and 2t + 2 (tile t + 1)
      auto tile = [&](auto par, auto masking, int t) __attribute__((always_inline)) {
        constexpr int PT = decltype(par)::value;
        // page ids first: their scalar loads overlap the wait for the other waves
        const int32_t kp = fwd_page(walk, min(t + 2, n_tiles - 1), wave);
        const int32_t vp = fwd_page(walk, t + 1, wave);
        wait_vmcnt<0>();
        barrier();
        if (t + 2 < n_tiles) load_page<D, kSwzRow>(kh, kp, (lds_char *)(PT ? kbuf1 : kbuf0), 16 * wave, lane);
        load_page<D, kSwzTr>(vh, vp, (lds_char *)(PT ? vbuf0 : vbuf1), 16 * wave, lane);
        const lds_char *knext = PT ? K0 : K1;  // K_{t+1}
        const lds_char *vcur = PT ? V1 : V0;   // V_t
        step(T, T, ic<1>{}, masking, knext, vcur, 2 * t + 1);
        step(T, T, ic<0>{}, masking, knext, vcur, 2 * t + 2);
      };
      // bodies t < full_tiles - 1 touch only tiles of the valid prefix
      const int split = min(max(full_tiles - 1, 0), n_tiles - 1);
      for_range(ic<kMaskNone>{}, 0, split, tile);
      for_range(ic<kMaskAlways>{}, split, n_tiles - 1, tile);
      // last tile t = n_tiles - 1: V_t resident after the wait
      const int t = n_tiles - 1;
      wait_vmcnt<0>();
      barrier();
      const lds_char *vlast = (t & 1) ? V1 : V0;
      step(F, T, ic<1>{}, ic<kMaskCheck>{}, K0, vlast, 2 * t + 1);
      rescale();
      pv(vlast, 1, pacc[1]);
    } else {
      // One sub-tile per tile.  Before sub-iteration i: K_{i+1} and V_{i-1} resident;
      // then K_{i+2} goes into the buffer of K_i and V_i into the buffer of V_{i-2}.
      if (n_tiles > 1) wait_vmcnt<LOADS>(); else wait_vmcnt<0>();
      barrier();
      qk(K0, 0, sacc[0]);
      wait_vmcnt<0>();
      barrier();
      if (n_sub > 2) load_page<D, kSwzRow>(kh, fwd_page(walk, 2, wave), (lds_char *)kbuf0, 16 * wave, lane);
      load_page<D, kSwzTr>(vh, fwd_page(walk, 0, wave), (lds_char *)vbuf0, 16 * wave, lane);
      if (n_sub > 1) {
        step(T, F, ic<0>{}, ic<kMaskCheck>{}, K1, V1, 0);
        nm_fix = m2 == kNegInf ? 0.f : -m2;
        auto sub = [&](auto par, auto masking, int i) __attribute__((always_inline)) {
          constexpr int PI = decltype(par)::value;
          const int32_t kp = fwd_page(walk, min(i + 2, n_sub - 1), wave);
          const int32_t vp = fwd_page(walk, i, wave);
          wait_vmcnt<0>();
          barrier();
          if (i + 2 < n_sub) load_page<D, kSwzRow>(kh, kp, (lds_char *)(PI ? kbuf1 : kbuf0), 16 * wave, lane);
          load_page<D, kSwzTr>(vh, vp, (lds_char *)(PI ? vbuf1 : vbuf0), 16 * wave, lane);
          step(T, T, par, masking, PI ? K0 : K1, PI ? V0 : V1, i);
        };
        const int split = min(max(full_tiles, 1), n_sub - 1);
        for_range(ic<kMaskNone>{}, 1, split, sub);
        for_range(ic<kMaskAlways>{}, split, n_sub - 1, sub);
        // last sub-iteration i = n_sub - 1
        const int i = n_sub - 1;
        wait_vmcnt<0>();
        barrier();
        load_page<D, kSwzTr>(vh, fwd_page(walk, i, wave), (lds_char *)((i & 1) ? vbuf1 : vbuf0), 16 * wave, lane);
        if (i & 1) step(F, T, ic<1>{}, ic<kMaskCheck>{}, K0, V0, i);
        else step(F, T, ic<0>{}, ic<kMaskCheck>{}, K0, V1, i);
      } else {
        step(F, F, ic<0>{}, ic<kMaskCheck>{}, K1, V1, 0);
      }
      rescale();
      wait_vmcnt<0>();
      barrier();
      if ((n_sub - 1) & 1) pv(V1, 0, pacc[1]); else pv(V0, 0, pacc[0]);
    }
  }

  // ---- merge the waves that share query rows, then write O and LSE ----
  wait_vmcnt<0>();
  if (!EXACT && tid == 0) redo_any = 0;
  // fast kernel: the fixed maximum is only safe if it existed before the row's first
  // probability (else the sums ran against 0) and no score rose more than 2^kLimit
  // above it (every probability is at most the row sum)
  if (!EXACT) over = over || (m2 == kNegInf && l_run != 0.f) || !(l_run <= __builtin_exp2f(kLimit));
  // s_barrier does not wait for LDS writes on this GPU: the reset of the flag (and every
  // LDS read of the loop) completes before any wave can pass and set it
  wait_lgkm0();
  barrier();
  if (!EXACT && __builtin_amdgcn_ballot_w64(over) != 0 && lane == 0) redo_any = 1;
  {
    const float lt = l_run + __shfl_xor(l_run, 32);
    if (lane < 32) {
      stat_m[wave][l32] = m2;
      stat_l[wave][l32] = lt;
    }
  }
  wait_lgkm0();
  barrier();
  const int64_t orow0 = (int64_t)bh * args.seq_q + 128 * item_block0(it, args.groups);
  if (!EXACT && redo_any) {
    // the exact kernel writes this item; the mark lives in the caller's own LSE row,
    // so concurrent calls on one plan (different outputs) never see each other's
    if (tid == 0) args.lse[orow0] = __builtin_bit_cast(float, kRedoMark);
    return;
  }
  // merged maximum and sum of query row qr (0..31) of query group q_g
  auto merged = [&](int q_g, int qr, float *mt_out) __attribute__((always_inline)) -> float {
    float mt = kNegInf;
#pragma unroll
    for (int w = q_g; w < kWaves; w += NQG) mt = fmaxf(mt, stat_m[w][qr]);
    float lt = 0.f;
#pragma unroll
    for (int w = q_g; w < kWaves; w += NQG)
      if (stat_m[w][qr] != kNegInf) lt += stat_l[w][qr] * __builtin_amdgcn_exp2f(stat_m[w][qr] - mt);
    *mt_out = mt;
    return lt;
  };
  // per-wave fp32 partial output (32 rows x D) over the free tile buffers
  constexpr int PART_BYTES = 32 * D * 4;
  {
    float mt;
    const float lt = merged(qg, l32, &mt);
    const float f = (m2 == kNegInf || lt == 0.f) ? 0.f : __builtin_amdgcn_exp2f(m2 - mt) / lt;
    lds_char *part = (lds_char *)smem + wave * PART_BYTES;
#pragma unroll
    for (int n = 0; n < ND; ++n) {
      const f32x16 o = oacc[n] * f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c4 = 8 * n + 2 * j + g;                  // float4 chunk of d = 32n + 8j + 4g
        const int phys = c4 ^ (l32 & (D / 4 - 1));
        const f32x4 val = {o[4 * j], o[4 * j + 1], o[4 * j + 2], o[4 * j + 3]};
        *(__attribute__((address_space(3))) f32x4 *)(part + (l32 * D + 4 * phys) * 4) = val;
      }
    }
  }
  wait_lgkm0();
  barrier();

  // Output spans: a plain item writes the 128 rows of its block (valid rows from the
  // waves of their query group, the rest O = 0, LSE = -inf); a group item writes the 128
  // rows of each member block, member m's valid rows from wave m.
  const bool grouped = ROUTE == 128 && it.q < 0;
  const int n_spans = grouped ? NQG : 1;
  int32_t span_q[NQG], span_rows[NQG];
  if (grouped) {
    const FwdGroup &gr = args.groups[~it.q];
#pragma unroll
    for (int m = 0; m < NQG; ++m) {
      span_q[m] = gr.q[m];
      span_rows[m] = gr.c_q[m];
    }
  } else {
#pragma unroll
    for (int m = 0; m < NQG; ++m) {
      span_q[m] = it.q;
      span_rows[m] = it.c_q < M ? it.c_q : M;
    }
  }
  // span m, row r: (block, valid, query group, row inside the group)
  auto span_row = [&](int m, int r, int *blk, int *q_g, int *qr) __attribute__((always_inline)) -> bool {
    *blk = span_q[m];
    if (grouped) {
      *q_g = m;
      *qr = r;
    } else {
      *q_g = r >> 5;
      *qr = r & 31;
    }
    return *blk >= 0 && r < span_rows[m];
  };
  constexpr int GROUPS = D / 8;
  for (int u = tid; u < n_spans * 128 * GROUPS; u += kThreads) {
    const int m = u / (128 * GROUPS), row = (u / GROUPS) & 127, grp = u % GROUPS;
    int blk, q_g, qr;
    const bool valid = span_row(m, row, &blk, &q_g, &qr);
    if (blk < 0) continue;  // a group item without member m
    float acc8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (valid) {
      for (int w = q_g; w < kWaves; w += NQG) {
        const lds_char *pw = (const lds_char *)smem + w * PART_BYTES;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int phys = (2 * grp + h) ^ (qr & (D / 4 - 1));
          const f32x4 x = *(const __attribute__((address_space(3))) f32x4 *)(pw + (qr * D + 4 * phys) * 4);
          acc8[4 * h] += x[0];
          acc8[4 * h + 1] += x[1];
          acc8[4 * h + 2] += x[2];
          acc8[4 * h + 3] += x[3];
        }
      }
    }
    bf16x8 out;
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (__bf16)acc8[e];
    const int64_t orow = (int64_t)bh * args.seq_q + 128 * blk + row;
    *(bf16x8 *)((char *)args.o + (orow * D + 8 * grp) * 2) = out;
  }
  for (int u = tid; u < n_spans * 128; u += kThreads) {
    const int m = u >> 7, row = u & 127;
    int blk, q_g, qr;
    const bool valid = span_row(m, row, &blk, &q_g, &qr);
    if (blk < 0) continue;
    float lse = kNegInf;
    if (valid) {
      float mt;
      const float lt = merged(q_g, qr, &mt);
      // LSE = ln(sum exp(scale * s)) = (m2 + log2 l) * ln 2
      if (mt != kNegInf && lt > 0.f) lse = (mt + __log2f(lt)) * 0.6931471805599453f;
    }
    args.lse[(int64_t)bh * args.seq_q + 128 * blk + row] = lse;
  }
}

// Both routes in one launch: workgroup b runs M128 x N128 item order[b] when that is
// >= 0, else M64 x N256 item ~order[b] (or a cleanup item of an empty block); without an
// order table the M128 items come first.  Per head the M64 items follow the M128 items,
// so they fill the end of that work and find its pages in the caches.
template <int D>
__global__ __launch_bounds__(kThreads, 2) void kpage_fwd_kernel(FwdArgs a128, FwdArgs a64) {
  __shared__ FwdLds<D> lds;
  const int b = blockIdx.x;
  const int t = a128.order ? a128.order[b] : (b < a128.n_items ? b : ~(b - a128.n_items));
  if (t >= 0) {
    if (a128.route_only != 64) fwd_item<D, 128, false>(a128, t, lds);
  } else if (a128.route_only != 128) {
    fwd_item<D, 64, false>(a64, ~t, lds);
  }
}

// Exact re-run over the items the fast kernel marked (first LSE row = kRedoMark): a small
// grid whose workgroups check 256 items at a time (one per thread) and run the marked
// ones, so a launch with nothing marked costs a few microseconds.
template <int D>
__global__ __launch_bounds__(kThreads, 2) void kpage_fwd_exact_kernel(FwdArgs a128, FwdArgs a64) {
  __shared__ FwdLds<D> lds;
  __shared__ uint64_t marked[kWaves];
  const int n = a128.n_items + a64.n_items;
  const int tid = threadIdx.x;
  for (int base = blockIdx.x * kThreads; base < n; base += gridDim.x * kThreads) {
    const int i = base + tid;
    bool mark = false;
    if (i < n) {
      const FwdItem it = i < a128.n_items ? a128.items[i] : a64.items[i - a128.n_items];
      mark = __builtin_bit_cast(uint32_t, a128.lse[(int64_t)it.bh * a128.seq_q + 128 * item_block0(it, a128.groups)]) ==
             kRedoMark;
    }
    const uint64_t m = __builtin_amdgcn_ballot_w64(mark);
    if ((tid & 63) == 0) marked[tid >> 6] = m;
    __syncthreads();
    for (int w = 0; w < kWaves; ++w) {
      const uint64_t mw = marked[w];
      uint64_t left = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(mw >> 32)) << 32) |
                      __builtin_amdgcn_readfirstlane((uint32_t)mw);
      while (left) {
        const int j = base + 64 * w + __builtin_ctzll(left);
        left &= left - 1;
        if (j < a128.n_items) fwd_item<D, 128, true>(a128, j, lds);
        else fwd_item<D, 64, true>(a64, j - a128.n_items, lds);
        __syncthreads();  // the next item reuses the LDS
      }
    }
    __syncthreads();  // `marked` is rewritten by the next round
  }
}

template <int D>
void launch_d(const FwdArgs &a128, const FwdArgs &a64, hipStream_t stream, LaunchTimer *timer) {
  dim3 grid(a128.n_items + a64.n_items), block(kThreads);
  if (timer && timer->split_routes()) {
    // profiling: the full launch twice, each running one route's items at the launch
    // positions they hold in the combined launch (the other route's workgroups exit)
    FwdArgs only128 = a128, only64 = a128;
    only128.route_only = 128;
    only64.route_only = 64;
    timer->before(KPAGE_K_FWD, stream);
    hipLaunchKernelGGL((kpage_fwd_kernel<D>), grid, block, 0, stream, only128, a64);
    timer->after(KPAGE_K_FWD, stream);
    timer->before(KPAGE_K_FWD_Q64, stream);
    hipLaunchKernelGGL((kpage_fwd_kernel<D>), grid, block, 0, stream, only64, a64);
    timer->after(KPAGE_K_FWD_Q64, stream);
  } else {
    if (timer) timer->before(KPAGE_K_FWD, stream);
    hipLaunchKernelGGL((kpage_fwd_kernel<D>), grid, block, 0, stream, a128, a64);
    if (timer) timer->after(KPAGE_K_FWD, stream);
  }
  const int n = a128.n_items + a64.n_items;
  const int exact_blocks = std::min((n + kThreads - 1) / kThreads, kExactBlocks);
  if (timer) timer->before(KPAGE_K_FWD_EXACT, stream);
  hipLaunchKernelGGL((kpage_fwd_exact_kernel<D>), dim3(exact_blocks), block, 0, stream, a128, a64);
  if (timer) timer->after(KPAGE_K_FWD_EXACT, stream);
}

}  // namespace

hipError_t launch_fwd(const FwdArgs &a128, const FwdArgs &a64, int head_dim, hipStream_t stream,
                      LaunchTimer *timer) {
  if (a128.n_items < 0 || a64.n_items < 0) return hipErrorInvalidValue;
  if (a128.n_items + a64.n_items == 0) return hipSuccess;
  if (head_dim == 128) launch_d<128>(a128, a64, stream, timer);
  else if (head_dim == 64) launch_d<64>(a128, a64, stream, timer);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace kpage
