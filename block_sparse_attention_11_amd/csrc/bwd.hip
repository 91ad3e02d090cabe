// Backward KPage attention for gfx950 (MI355X, CDNA4).
//
// KPage paper, section 3.3: dK and dV are accumulated by K/V owners.  An owner is
// 8 Page16 slots (128 key rows) holding pages of one or more logical K/V blocks;
// no block crosses an owner.  Its reverse-Q neighbourhood is visited in steps of 8
// query pages (128 query rows), and one 64-bit adjacency word per step (bit 8 j + i:
// Q slot j, K slot i) removes the page pairs that are not edges of the original
// graph (section 3.3.3).
//
// dQ is computed by a second, Q-owned pass over the forward page walks (section
// 3.2): each query block recomputes S and dP for its own keys and accumulates
// dQ = scale dS K in registers, so no query row is written by more than one
// workgroup and no fp32 accumulator or atomic traffic is needed.  This costs one
// more S and dP product per pair than an atomic dQ inside the owner loop, but on
// MI355X the owner loop would otherwise spend its LDS bandwidth on transposed dS
// and K reads and its memory bandwidth on fp32 atomics.
//
// Kernels, in launch order:
//   kpage_bwd_zero  zero dK/dV pages that lie outside every block footprint.
//   kpage_bwd_dq    one workgroup per forward work item (query block), both routes
//                   in one launch: dQ; its prologue also writes the row statistics
//                   D_i = sum_d dO_id O_id and LSE_i * log2(e) (+inf for rows without
//                   keys and rows past c_q) of the item's rows.
//   kpage_bwd_kv    one workgroup per (batch*head, owner), or per (batch*head,
//                   owner, Q group) when the plan splits reverse neighbourhoods
//                   into Q groups (section 3.3.2): dK, dV, or fp32 partials of them;
//                   reads the row statistics.
//   kpage_bwd_kv_reduce  sums the partials of owners split over Q groups.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "kpage.h"
#include "tile_common.hpp"

namespace kpage {
namespace {

// zero dK/dV on pages outside every block footprint: one block per (bh, page)
template <int D>
__global__ __launch_bounds__(256) void kpage_bwd_zero(BwdArgs a, int64_t pages_per_bh) {
  const int64_t bh = blockIdx.x / pages_per_bh;
  const int64_t i = blockIdx.x % pages_per_bh;
  const int slot = a.per_head ? (int)bh : 0;
  const int64_t n = a.uncovered_ptr[slot + 1] - a.uncovered_ptr[slot];
  if (i >= n) return;
  const int64_t page = a.uncovered[a.uncovered_ptr[slot] + i];
  const int64_t base = (bh * a.seq_kv + page * 16) * D;
  for (int e = threadIdx.x * 8; e < 16 * D; e += 256 * 8) {
    *(bf16x8 *)((__bf16 *)a.dk + base + e) = bf16x8{};
    *(bf16x8 *)((__bf16 *)a.dv + base + e) = bf16x8{};
  }
}

// ---------------------------------------------------------------------------
// K/V-owned pass.  One workgroup of 4 waves per (b*h, owner), two workgroups per CU
// (so the two waves sharing a SIMD belong to different workgroups and drift apart:
// one's element-wise work overlaps the other's MFMAs).  Wave w owns key rows
// 32 w .. + 31 of the owner (owner slots 2 w, 2 w + 1): its K and V rows stay in
// VGPRs as MFMA B operands and its dK and dV are accumulators.  Each 8-page query
// step runs as two half-steps of 4 Q pages (64 query rows), double-buffered in LDS.
//
// Per 32-query block: S = Q K^T and dP = dO V^T with the lane index over keys and
// the register index over queries (A = Q / dO rows read from LDS), so P^T and
// dS^T are directly the A operands of dV += P^T dO and dK += dS^T Q, whose B
// operands (columns of dO and Q) are transposed LDS reads of the same tiles.
constexpr int kKvWaves = 4;

template <int D>
__global__ __launch_bounds__(64 * kKvWaves, 2) void kpage_bwd_kv(BwdArgs a) {
  constexpr int DS = D / 16;
  constexpr int ND = D / 32;
  constexpr int TILE = 64 * D * 2;        // one half-step tile (4 pages) of Q or dO
  constexpr int STATS = kKvWaves * 256;   // per half-step: 64 floats per page (lse2, delta, spare)

  // half-step buffers [Q 0][dO 0][Q 1][dO 1] (every offset fits a ds_read immediate)
  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE];
  __shared__ __attribute__((aligned(256))) char stats[2 * STATS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // key group: slots 2 w, 2 w + 1
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int sl = lane & 15;
  const int mgrp = lane >> 4;
  const int khalf = l32 >> 4;

  const BwdItem it = a.items[blockIdx.x];
  const int64_t bh = it.bh;
  const int n_half = 2 * it.n_steps;
  c_i32 *own = (c_i32 *)(a.owners + (int64_t)it.owner * 8);
  c_u32 *kmk = (c_u32 *)(a.owner_kmask + (int64_t)it.owner * 8);
  c_i32 *qpages = (c_i32 *)(a.qpages + it.qwalk_off);
  c_u64 *adjw = (c_u64 *)(a.adj + (it.qwalk_off >> 3));

  const char *kh = (const char *)a.k + bh * a.seq_kv * D * 2;
  const char *vh = (const char *)a.v + bh * a.seq_kv * D * 2;
  const char *qgl = (const char *)a.q + bh * a.seq_q * D * 2;
  const char *ggl = (const char *)a.dout + bh * a.seq_q * D * 2;
  const float *l2h = a.lse2 + bh * a.seq_q;
  const uint32_t stat_off =
      (uint32_t)(lane & 15) * 4 + ((lane >> 4) & 1) * (uint32_t)((const char *)a.delta - (const char *)a.lse2);

  // half-step u (pages 4 (u & 1) .. + 3 of step u / 2): one Q and one dO page per wave,
  // and the page's lse2 and delta
  auto load_half = [&](int32_t page, auto buf_c) __attribute__((always_inline)) {
    constexpr int buf = decltype(buf_c)::value;
    lds_char *qt = (lds_char *)smem + (2 * buf) * TILE;
    lds_char *gt = (lds_char *)smem + (2 * buf + 1) * TILE;
    load_page<D, kSwzBoth>(qgl, page, qt, 16 * wave, lane);
    load_page<D, kSwzBoth>(ggl, page, gt, 16 * wave, lane);
    // lanes 0-15: lse2 of the page's rows, 16-31: delta, 32-63: the same again
    // (delta = lse2 + rows: one scalar base and a 32-bit lane offset)
    const char *src = (const char *)(l2h + (int64_t)page * 16);
    const uint32_t off = (uint32_t)xor_imm<0x40000000>(stat_off) ^ 0x40000000u;  // recomputed, not kept
    lds_dma<4>(src, off, (lds_char *)(stats + buf * STATS + wave * 256));
  };

  // this wave's 32 key rows as MFMA B operands (k = head dim, n = key).  Empty owner
  // slots read finite data of slot 0; their results are never stored.
  bf16x8 kreg[DS], vreg[DS];
  {
    const int32_t page_raw = own[2 * wave + khalf];
    const int32_t page = page_raw >= 0 ? page_raw : own[0];
    const bf16x8 *kr = (const bf16x8 *)(kh + ((int64_t)page * 16 + (l32 & 15)) * (D * 2));
    const bf16x8 *vr = (const bf16x8 *)(vh + ((int64_t)page * 16 + (l32 & 15)) * (D * 2));
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      kreg[s] = kr[2 * s + g];
      vreg[s] = vr[2 * s + g];
    }
  }
  if (n_half > 0) load_half(qpages[wave], ic<0>{});

  f32x16 dk[ND], dv[ND];
#pragma unroll
  for (int n = 0; n < ND; ++n) {
    dk[n] = f32x16{};
    dv[n] = f32x16{};
  }
  const float c2 = a.scale_log2;
  // B operand of the extra dP k-step: ones in k = 0, 1 (lanes 0-31), zeros elsewhere
  const uint32_t ones_lo = g ? 0u : 0x3F803F80u;
  // Lane-constant LDS offsets inside a Q or dO tile.  Row reads of row l32 of a
  // 32-query block at k-step s sit at rd_base ^ 32 s (the swizzle only flips chunk
  // bits and repeats every 16 rows).  Transposed reads of rows tr_row and tr_row + 8
  // of a 16-row group at head-dim block n sit at tr_base ^ 64 n and at
  // (tr_base ^ 64 (n ^ 1)) + 8 rows (row + 8 flips chunk bit 2).  Query block,
  // buffer and tile are immediates.
  const int rd_base = chunk_off<kSwzBoth, D>(l32, g);
  const int tr_base = chunk_off<kSwzBoth, D>(4 * g + (sl >> 2), 2 * (mgrp & 1) + ((sl & 3) >> 1)) + (sl & 1) * 8;

  // Lane parts of the lse2 / delta reads with the stats buffer's own LDS address folded
  // in, kept opaque: every read is then this base plus a constant that fits the 16-bit
  // read offset (the buffer sits past the first 64 KiB of LDS).
  uint32_t st_lse = (uint32_t)(uintptr_t)(const lds_char *)stats + 16 * g;
  uint32_t st_del = (uint32_t)(uintptr_t)(const lds_char *)stats + ((l32 >> 4) * 64 + 16 + (l32 & 15)) * 4;
  asm volatile("" : "+v"(st_lse), "+v"(st_del));

  auto half_step = [&](auto buf_c, int u, uint64_t adj) __attribute__((always_inline)) {
    constexpr int BUF = decltype(buf_c)::value;
    const lds_char *qt = (const lds_char *)smem + (2 * BUF) * TILE;
    const lds_char *gt = (const lds_char *)smem + (2 * BUF + 1) * TILE;
    const lds_char *stl = (const lds_char *)(uintptr_t)st_lse + BUF * STATS;
    const lds_char *std_ = (const lds_char *)(uintptr_t)st_del + BUF * STATS;
    // Pair mask.  Query rows without a valid key (invalid rows included) have
    // lse2 = +inf, so their P is 0 by itself.  Key validity needs no mask here: the P
    // and dS of an invalid key reach only that key's own dK / dV rows, which are
    // written as 0.  What is left is the adjacency bit of (query page, key slot); it
    // is all ones on almost every step, so the zeroing of non-edge P blocks runs in a
    // wave-uniform branch.  The 2 bits of this wave's slots for page j sit at bit
    // 8 (4 (u & 1) + j) + 2 w of the step's word.
    const int jbase = 4 * (u & 1);
    uint32_t nib = 0xFFu;  // 2 bits per page of the half-step
#pragma unroll
    for (int j = 0; j < 4; ++j) nib &= ~((~(uint32_t)(adj >> (8 * (jbase + j) + 2 * wave)) & 0x3u) << (2 * j));
    const bool all_edges = nib == 0xFFu;
    // the first two Q-row operands of the next query block's S chain
    bf16x8 qpre[2];
    qpre[0] = lds_read8(qt + xor_imm<0>(rd_base));
    qpre[1] = lds_read8(qt + xor_imm<32>(rd_base));
    __builtin_amdgcn_sched_barrier(0);
    static_for<2>([&](auto qb_c) __attribute__((always_inline)) {
      constexpr int QB = decltype(qb_c)::value;
      constexpr int RB = 32 * QB * D * 2;  // byte offset of the query block
      // Register r of a 32 x 32 score block holds query row 32 qb + 8 (r / 4) + 4 g +
      // r % 4 of the half-step; group j4 = r / 4 reads its 4 lse2 values as one f32x4.
      auto lse4 = [&](int j4) __attribute__((always_inline)) {
        // q = 32 qb + 8 j4 + 4 g: page 2 qb + j4 / 2, row 8 (j4 % 2) + 4 g (4 g is in stl)
        return *(const __attribute__((address_space(3))) f32x4 *)(stl + ((2 * QB + (j4 >> 1)) * 64 + 8 * (j4 & 1)) * 4);
      };
      auto rd_row = [&](const lds_char *t, auto s_c) __attribute__((always_inline)) {
        constexpr int S = decltype(s_c)::value;
        return lds_read8(t + RB + xor_imm<32 * S>(rd_base));
      };
      // The block is one stream of MFMAs: S = Q K^T (DS), dP - D = dO V^T - D (DS + 1),
      // dV += P^T dO and dK += dS^T Q (2 ND each half).  The element-wise work sits
      // between them where its inputs are ready and its outputs are not yet needed, so a
      // wave's VALU and MFMA work overlap: the probabilities of group j4 (4 scores per
      // lane) between the dP MFMAs, the dS of the first 16 queries between the first dV
      // MFMAs, that of the other 16 between the first dK MFMAs.  Row operands are read
      // from LDS two MFMAs ahead across the S -> dP boundary, each lse2 group two MFMAs
      // before its use.
      // P slice j4 sits after dP MFMA p_at(j4) (-1: right after the S chain, which frees
      // half of the score registers before the dP chain: the register file has no room
      // for all of S and dP at once)
      constexpr int p_at[4] = {-1, -1, DS == 8 ? 2 : 1, DS == 8 ? 5 : 3};
      f32x16 sp, dp;
      f32x4 l4[4];
      float nd = 0.f;
      u32x4 pb[2], sb[2];  // P and dS as packed bf16 pairs (u32x4 [hh] = rows 16 hh .. + 15)
      bf16x8 op[2 * DS];   // S chain operands (Q rows), then dP chain operands (dO rows)
      op[0] = qpre[0];
      op[1] = qpre[1];
      auto read_op = [&](auto i_c) __attribute__((always_inline)) {
        constexpr int I = decltype(i_c)::value;
        if constexpr (I < DS) op[I] = rd_row(qt, ic<I>{});
        else if constexpr (I < 2 * DS) op[I] = rd_row(gt, ic<I - DS>{});
      };
      // (A) S = Q K^T
      static_for<DS>([&](auto s_c) __attribute__((always_inline)) {
        constexpr int S = decltype(s_c)::value;
        read_op(ic<S + 2>{});
        if constexpr (S == DS - 2) nd = -*(const __attribute__((address_space(3))) float *)(
                                        std_ + 2 * QB * 64 * 4);
        if constexpr (S == DS - 4) l4[0] = lse4(0);
        if constexpr (S == DS - 3) l4[1] = lse4(1);
        sp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[S], kreg[S], S == 0 ? f32x16{} : sp, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      });
      // P = exp2(scale log2e S - lse2) for score group j4
      auto p_slice = [&](auto j_c) __attribute__((always_inline)) {
        constexpr int J4 = decltype(j_c)::value;
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
          const int r = 4 * J4 + e;
          pb[r >> 3][(r & 7) >> 1] =
              pinned(pack_bf16(__builtin_amdgcn_exp2f(__builtin_fmaf(sp[r], c2, -l4[J4][e])),
                               __builtin_amdgcn_exp2f(__builtin_fmaf(sp[r + 1], c2, -l4[J4][e + 1]))));
        }
      };
      p_slice(ic<0>{});
      p_slice(ic<1>{});
      __builtin_amdgcn_sched_barrier(0);
      // (B) dP - D = dO V^T - D, with D as one extra k-step (A = -D split into bf16 hi +
      // lo in k = 0, 1 of lanes 0-31 for query row l32, B = ones), then dS = P (dP - D)
      // with P as its bf16 value (an extra rounding of the order of dS's own)
      static_for<DS>([&](auto s_c) __attribute__((always_inline)) {
        constexpr int S = decltype(s_c)::value;
        read_op(ic<DS + S + 2>{});
        if constexpr (S == 0) l4[2] = lse4(2);
        if constexpr (S == p_at[3] - 2) l4[3] = lse4(3);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[DS + S], vreg[S], S == 0 ? f32x16{} : dp, 0, 0, 0);
        static_for<4>([&](auto j_c) __attribute__((always_inline)) {
          if constexpr (p_at[decltype(j_c)::value] == S) p_slice(j_c);
        });
        __builtin_amdgcn_sched_barrier(0);
      });
      {
        const float hi = __builtin_bit_cast(float, pack_bf16(nd, 0.f) << 16);
        const bf16x8 daug = __builtin_bit_cast(bf16x8, u32x4{g ? 0u : pack_bf16(hi, nd - hi), 0u, 0u, 0u});
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(daug, __builtin_bit_cast(bf16x8, u32x4{ones_lo, 0u, 0u, 0u}), dp,
                                                     0, 0, 0);
      }
      // zero the P blocks of non-edge (query page, key slot) pairs: pb[hh] holds the
      // rows of page 2 qb + hh of the half-step
      if (!all_edges) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          if (!((nib >> (2 * (2 * QB + hh) + khalf)) & 1u)) pb[hh] = u32x4{};
      }
      __builtin_amdgcn_sched_barrier(0);
      // (C) dV += P^T dO and dK += dS^T Q over these 32 query rows, in the operand order
      // dV (hh 0), dK (hh 0), dV (hh 1), dK (hh 1); B operands = columns of dO and Q,
      // transposed reads one product ahead.  The next query block's first Q rows are
      // read during the last products.
      constexpr int NOPS = 4 * ND;
      bf16x8 top[NOPS];
      // the ND lane offsets tr_base ^ 64 n of this block's transposed reads, computed
      // once for its 4 ND operands (8 ND reads)
      int trx[ND];
      static_for<ND>([&](auto n_c) __attribute__((always_inline)) {
        trx[decltype(n_c)::value] = xor_imm<64 * decltype(n_c)::value>(tr_base);
      });
      // operand i: tile (dO for even phase, Q for odd), hh = i / (2 ND), n = i % ND
      auto rdt = [&](auto i_c) __attribute__((always_inline)) {
        constexpr int I = decltype(i_c)::value;
        if constexpr (I < NOPS) {
          constexpr int PH = I / ND, N = I % ND, HH = PH / 2;
          constexpr int RH = RB + 16 * HH * D * 2;
          const lds_char *t = (PH & 1) ? qt : gt;
          top[I] = tr_read8(t + RH + trx[N], t + RH + 8 * D * 2 + trx[N ^ 1]);
        }
      };
      auto ds_pair = [&](auto r_c) __attribute__((always_inline)) {
        constexpr int R = decltype(r_c)::value;
        const uint32_t w = pb[R >> 3][(R & 7) >> 1];
        sb[R >> 3][(R & 7) >> 1] = pinned(pack_bf16(__builtin_bit_cast(float, w << 16) * dp[R],
                                                    __builtin_bit_cast(float, w & 0xFFFF0000u) * dp[R + 1]));
      };
      rdt(ic<0>{});
      rdt(ic<1>{});
      __builtin_amdgcn_sched_barrier(0);
      static_for<NOPS>([&](auto i_c) __attribute__((always_inline)) {
        constexpr int I = decltype(i_c)::value;
        constexpr int PH = I / ND, N = I % ND, HH = PH / 2;
        rdt(ic<I + 2>{});
        if constexpr (QB == 0 && I == NOPS - 2) {
          qpre[0] = lds_read8(qt + RB + 32 * D * 2 + xor_imm<0>(rd_base));
          qpre[1] = lds_read8(qt + RB + 32 * D * 2 + xor_imm<32>(rd_base));
        }
        if constexpr ((PH & 1) == 0)
          dv[N] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, pb[HH]), top[I], dv[N], 0, 0, 0);
        else
          dk[N] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, sb[HH]), top[I], dk[N], 0, 0, 0);
        // dS of rows 16 hh .. + 15 (4 pairs) during the phase before its first use:
        // hh 0 during dV (hh 0), hh 1 during dK (hh 0)
        if constexpr (PH < 2) {
          constexpr int HHS = PH;  // rows being computed
          if constexpr (ND == 4) ds_pair(ic<8 * HHS + 2 * N>{});
          else { ds_pair(ic<8 * HHS + 4 * N>{}); ds_pair(ic<8 * HHS + 4 * N + 2>{}); }
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    });
  };

  // one half-step per iteration; the next one's pages load while this one computes
  auto iter = [&](auto buf_c, auto, int u) __attribute__((always_inline)) {
    constexpr int BUF = decltype(buf_c)::value;
    // scalar table reads first and complete, so that no scalar load is in flight
    // while the LDS reads of the half-step wait on their counter
    const int32_t pn = qpages[4 * min(u + 1, n_half - 1) + wave];
    const uint64_t adj = adjw[u >> 1];
    wait_lgkm0();
    wait_vmcnt<0>();
    barrier();  // half-step u resident for every wave; nobody reads buffer 1 - BUF any more
    if (u + 1 < n_half) load_half(pn, ic<1 - BUF>{});
    // A half-step with no edge between its 4 query pages and this wave's 2 key slots
    // (dummy query pages, or pages of blocks outside each other's selection) has P = 0
    // and dS = 0 everywhere and adds nothing to dK and dV: the wave skips its compute
    // (wave-uniform; the copies above and the barriers are unchanged).
    const uint64_t wave_bits = (0x03030303ull << (32 * (u & 1))) << (2 * wave);
    if ((adj & wave_bits) != 0) half_step(buf_c, u, adj);
  };
  for_range(ic<0>{}, 0, n_half, iter);

  // ---- write dK (scaled) and dV by page id ----
  // lane = head-dim column, register r = key row acc_row(r, g) of the wave's 32 keys
  if (it.partial >= 0) {  // one of several Q groups of this owner: unscaled fp32 partials
    float *pk = a.part + (int64_t)it.partial * 2 * 128 * D + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 32 * wave + acc_row(r, g);
#pragma unroll
      for (int n = 0; n < ND; ++n) {
        pk[key * D + 32 * n] = dk[n][r];
        pk[(128 + key) * D + 32 * n] = dv[n][r];
      }
    }
    return;
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int key = 32 * wave + acc_row(r, g);
    const int slot = key >> 4, rin = key & 15;
    const uint32_t km = kmk[slot];
    if (km == 0u) continue;  // empty owner slot
    const int64_t page = own[slot];
    const bool ok = (km >> rin) & 1u;
    __bf16 *kdst = (__bf16 *)a.dk + (bh * a.seq_kv + page * 16 + rin) * D + l32;
    __bf16 *vdst = (__bf16 *)a.dv + (bh * a.seq_kv + page * 16 + rin) * D + l32;
#pragma unroll
    for (int n = 0; n < ND; ++n) {
      kdst[32 * n] = (__bf16)(ok ? dk[n][r] * a.scale : 0.f);
      vdst[32 * n] = (__bf16)(ok ? dv[n][r] : 0.f);
    }
  }
}

// ---------------------------------------------------------------------------
// Q-owned dQ pass over the forward page walks.  One workgroup of 4 waves per forward
// work item (query block), two workgroups per CU; the walk is consumed in half-tiles
// of 4 pages (64 keys), double-buffered in LDS, one K and one V page per wave.  Each
// wave owns 32 query rows and a key range of every half-tile (M128: 4 query groups,
// all 64 keys as two 32-key sub-tiles; M64: 2 query groups x 2 key halves, one
// sub-tile).  Per sub-tile, in the forward's transposed layout (lane = query):
//   S^T = K Q^T, dP^T = V dO^T  (A = K / V rows from LDS, B = Q / dO rows in VGPRs),
//   P^T = exp2(scale log2e S^T - lse2), dS^T = P^T (dP^T - D),
//   dQ^T += K^T dS^T            (A = K read transposed from LDS, B = dS^T).
// K tiles use the layout that serves both row and transposed reads.
constexpr int kDqWaves = 4;

template <int D, int ROUTE>
__device__ __forceinline__ void dq_item(const BwdArgs &a, const FwdItem *items, int item, char *smem) {
  constexpr int DS = D / 16;
  constexpr int ND = D / 32;
  constexpr int M = ROUTE;
  constexpr int NQG = M / 32;
  constexpr int NKG = kDqWaves / NQG;
  constexpr int KW = 64 / NKG;  // keys of a half-tile per wave
  constexpr int NH = KW / 32;
  constexpr int HTILE = 64 * D * 2;  // one half-tile of K or V
  constexpr int PART_BYTES = 32 * D * 4;
  static_assert(kDqWaves * PART_BYTES <= 4 * HTILE, "dQ partials reuse the tile buffers");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int sl = lane & 15;
  const int mgrp = lane >> 4;

  const FwdItem it = items[item];
  const int64_t bh = it.bh;
  const int n_half = (it.n_pages + 3) / 4;  // all-dummy half-tiles of the padding skipped
  const int full_half = it.n_full / 4;
  const int qg = wave % NQG;
  const int keyoff = (wave / NQG) * KW;

  const char *kh = (const char *)a.k + bh * a.seq_kv * D * 2;
  const char *vh = (const char *)a.v + bh * a.seq_kv * D * 2;
  c_i32 *walk = (c_i32 *)(a.pages + it.walk_off);
  // this wave's 32 query rows (a group item's wave holds the rows of its own member
  // block): Q and dO as MFMA B operands, lse2 and delta per lane
  const WaveRows wr = wave_rows(it, a.fgroups, qg);
  c_u32 *vwords = (c_u32 *)(a.valid + wr.valid_off);
  const int64_t qrow = bh * a.seq_q + 128 * wr.block + wr.row0 + l32;
  const bool qok = l32 < wr.rows;
  const bool idle = wr.rows <= 0;  // wave-uniform: no valid row in this query group
  bf16x8 qreg[DS], greg[DS];
  {
    const bf16x8 *qp = (const bf16x8 *)((const char *)a.q + qrow * D * 2);
    const bf16x8 *gp = (const bf16x8 *)((const char *)a.dout + qrow * D * 2);
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      qreg[s] = qok ? qp[2 * s + g] : bf16x8{};
      greg[s] = qok ? gp[2 * s + g] : bf16x8{};
    }
  }
  // D = rowsum(dO * O) and lse2 = LSE * log2(e) of this lane's query row, from the
  // caller's O and LSE; rows past c_q get D = 0 and lse2 = +inf whatever O and LSE hold
  // there, and so do rows whose LSE is -inf (no valid key): exp2(x - lse2) = 0.  The
  // K/V-owned pass, which runs after this one, reads them from the workspace: every
  // query block is an item of this pass (empty ones as cleanup items), and its items
  // cover every row of the query pages that the K/V-owned walks visit.
  float dsum = 0.f;
  if (qok) {
    const bf16x8 *op = (const bf16x8 *)((const char *)a.o + qrow * D * 2);
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      const bf16x8 ov = op[2 * s + g];
#pragma unroll
      for (int e = 0; e < 8; ++e) dsum = __builtin_fmaf((float)ov[e], (float)greg[s][e], dsum);
    }
  }
  dsum = half_sum(dsum);  // the other half of the row's head dimension sits in lane ^ 32
  const float lse = qok ? a.lse[qrow] : kNegInf;
  const float lse2 = lse == kNegInf ? __builtin_inff() : lse * kLog2e;
  // one lane per row (query groups repeat over key halves); a group item's wave without
  // a member block writes nothing
  if (keyoff == 0 && g == 0 && (it.q >= 0 || !idle)) {
    a.delta[qrow] = dsum;
    a.lse2[qrow] = lse2;
  }
  const float nlse2 = -lse2;
  // D enters the dP^T chain as one extra k-step: A = ones in k = 0, 1 (lanes 0-31),
  // B = -D of this lane's query split into bf16 hi + lo in k = 0, 1, so the chain
  // yields dP^T - D and dS^T = P^T (dP^T - D) costs one multiply per element
  bf16x8 one_aug, nd_aug;
  {
    const float nd = -dsum;
    const float hi = __builtin_bit_cast(float, pack_bf16(nd, 0.f) << 16);
    nd_aug = __builtin_bit_cast(bf16x8, u32x4{g ? 0u : pack_bf16(hi, nd - hi), 0u, 0u, 0u});
    one_aug = __builtin_bit_cast(bf16x8, u32x4{g ? 0u : 0x3F803F80u, 0u, 0u, 0u});
  }
  auto load_half = [&](int32_t page, int buf) __attribute__((always_inline)) {
    load_page<D, kSwzBoth>(kh, page, (lds_char *)smem + buf * HTILE, 16 * wave, lane);
    load_page<D, kSwzRow>(vh, page, (lds_char *)smem + (2 + buf) * HTILE, 16 * wave, lane);
  };
  if (n_half > 0) load_half(walk[wave], 0);

  f32x16 dq[ND];
#pragma unroll
  for (int n = 0; n < ND; ++n) dq[n] = f32x16{};
  const float c2 = a.scale_log2;
  // Lane-constant LDS offsets of this wave's key range (half-tile, buffer and
  // sub-tile are immediates): K rows (row l32, k-step s) at rdk ^ 32 s, V rows at
  // rdv ^ 32 s, transposed K rows tr_row / tr_row + 8 of a 16-row group at head-dim
  // block n at trk ^ 64 n and (trk ^ 64 (n ^ 1)) + 8 rows.
  const int rdk = keyoff * D * 2 + chunk_off<kSwzBoth, D>(l32, g);
  const int rdv = keyoff * D * 2 + chunk_off<kSwzRow, D>(l32, g);
  const int trk = keyoff * D * 2 + chunk_off<kSwzBoth, D>(4 * g + (sl >> 2), 2 * (mgrp & 1) + ((sl & 3) >> 1)) +
                  (sl & 1) * 8;

  // One 32-key sub-tile as one MFMA stream: S^T = K Q^T (DS), dP^T - D (DS + 1),
  // dQ^T += K^T dS^T (2 ND).  The probabilities of score group j4 (4 per lane) are
  // computed between the dP MFMAs (S is complete by then), dS of the first 16 keys
  // before the dQ MFMAs and that of the other 16 between the first half of them, so a
  // wave's VALU work overlaps its own MFMAs.  K and V row operands stream two MFMAs
  // ahead across the S -> dP boundary, the transposed K operands one ahead.
  // MASKED: invalid key rows (validity word of the sub-tile) get P = 0 (a select, not a
  // product: the P of a padded key row may be inf).
  auto sub_tile = [&](auto buf_c, auto h_c, auto masked_c, int u) __attribute__((always_inline)) {
    constexpr int BUF = decltype(buf_c)::value, H = decltype(h_c)::value;
    constexpr bool MASKED = decltype(masked_c)::value;
    constexpr int RB = 32 * H * D * 2;  // byte offset of the sub-tile in the wave's key range
    const lds_char *kt = (const lds_char *)smem + BUF * HTILE + RB;
    const lds_char *vt = (const lds_char *)smem + (2 + BUF) * HTILE + RB;
    // P slice j4 after dP MFMA p_at[j4]
    constexpr int p_at[4] = {DS == 8 ? 1 : 0, DS == 8 ? 3 : 1, DS == 8 ? 5 : 2, DS == 8 ? 7 : 3};
    f32x16 s_acc, dp_acc;
    bf16x8 op[2 * DS];
    auto read_op = [&](auto i_c) __attribute__((always_inline)) {
      constexpr int I = decltype(i_c)::value;
      if constexpr (I < DS) op[I] = lds_read8(kt + (rdk ^ (32 * I)));
      else if constexpr (I < 2 * DS) op[I] = lds_read8(vt + (rdv ^ (32 * (I - DS))));
    };
    uint32_t word = 0;
    if constexpr (MASKED) {
      word = vwords[2 * u + ((keyoff + 32 * H) >> 5)];
      // no key of the sub-tile is valid for this wave's rows (pages a group member did not
      // select, dummy pages): P and dS are 0, the sub-tile adds nothing to dQ
      if (word == 0u) return;
    }
    read_op(ic<0>{});
    read_op(ic<1>{});
    static_for<DS>([&](auto s_c) __attribute__((always_inline)) {
      constexpr int S = decltype(s_c)::value;
      read_op(ic<S + 2>{});
      s_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[S], qreg[S], S == 0 ? f32x16{} : s_acc, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    });
    // probabilities in place of the scores; register r holds key row acc_row(r, g) of
    // the sub-tile, whose validity bit (the sub-tile's word: two 16-bit page masks) is
    // wave-uniform in each lane half: a scalar lane mask selects p or 0
    auto p_slice = [&](auto j_c) __attribute__((always_inline)) {
      constexpr int J4 = decltype(j_c)::value;
      static_for<4>([&](auto e_c) __attribute__((always_inline)) {
        constexpr int R = 4 * J4 + decltype(e_c)::value;
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s_acc[R], c2, nlse2));
        if constexpr (MASKED) s_acc[R] = select_lanes(row_lane_mask<R>(word), p, 0.f);
        else s_acc[R] = p;
      });
    };
    static_for<DS>([&](auto s_c) __attribute__((always_inline)) {
      constexpr int S = decltype(s_c)::value;
      read_op(ic<DS + S + 2>{});
      dp_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[DS + S], greg[S], S == 0 ? f32x16{} : dp_acc, 0, 0, 0);
      static_for<4>([&](auto j_c) __attribute__((always_inline)) {
        if constexpr (p_at[decltype(j_c)::value] == S) p_slice(j_c);
      });
      __builtin_amdgcn_sched_barrier(0);
    });
    dp_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(one_aug, nd_aug, dp_acc, 0, 0, 0);
    constexpr int NOPS = 2 * ND;
    bf16x8 kop[NOPS];
    auto rdt = [&](auto j_c) __attribute__((always_inline)) {
      constexpr int J = decltype(j_c)::value, HH = J / ND, N = J % ND;
      if constexpr (J < NOPS) {
        const lds_char *p = kt + 16 * HH * D * 2;
        kop[J] = tr_read8(p + (trk ^ (64 * N)), p + 8 * D * 2 + (trk ^ (64 * (N ^ 1))));
      }
    };
    u32x4 ds[2];
    auto ds_pair = [&](auto r_c) __attribute__((always_inline)) {
      constexpr int R = decltype(r_c)::value;
      ds[R >> 3][(R & 7) >> 1] = pinned(pack_bf16(s_acc[R] * dp_acc[R], s_acc[R + 1] * dp_acc[R + 1]));
    };
    rdt(ic<0>{});
    rdt(ic<1>{});
    static_for<4>([&](auto i_c) __attribute__((always_inline)) { ds_pair(ic<2 * decltype(i_c)::value>{}); });
    __builtin_amdgcn_sched_barrier(0);
    static_for<NOPS>([&](auto j_c) __attribute__((always_inline)) {
      constexpr int J = decltype(j_c)::value, HH = J / ND, N = J % ND;
      rdt(ic<J + 2>{});
      dq[N] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[J], __builtin_bit_cast(bf16x8, ds[HH]), dq[N], 0, 0, 0);
      // dS of keys 16 .. 31 during the products of keys 0 .. 15
      if constexpr (HH == 0) {
        if constexpr (ND == 4) ds_pair(ic<8 + 2 * N>{});
        else { ds_pair(ic<8 + 4 * N>{}); ds_pair(ic<8 + 4 * N + 2>{}); }
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  auto iter = [&](auto buf_c, auto masked_c, int u) __attribute__((always_inline)) {
    constexpr int BUF = decltype(buf_c)::value;
    const int32_t pnext = walk[4 * min(u + 1, n_half - 1) + wave];
    wait_lgkm0();
    wait_vmcnt<0>();
    barrier();  // half-tile u resident; buffer 1 - BUF free
    if (u + 1 < n_half) load_half(pnext, 1 - BUF);
    // a query group without valid rows computes nothing (its dQ rows are written as 0);
    // the wave still copies its pages and meets every barrier
    if (!idle)
      static_for<NH>([&](auto h_c) __attribute__((always_inline)) { sub_tile(buf_c, h_c, masked_c, u); });
  };
  // half-tiles of the fully valid prefix, then the ones that may hold invalid key rows
  const int split = min(full_half, n_half);
  for_range(ic<false>{}, 0, split, iter);
  for_range(ic<true>{}, split, n_half, iter);

  // ---- sum the waves that share query rows, then write dQ = scale * acc (bf16) ----
  // The barrier alone does not order LDS accesses on this GPU (the compiler inserts no
  // wait before it): each wave first waits for its own copies and LDS reads, and for its
  // partial's writes before the second barrier, as the forward's merge does.
  wait_vmcnt<0>();
  wait_lgkm0();
  barrier();
  {
    lds_char *part = (lds_char *)smem + wave * PART_BYTES;
#pragma unroll
    for (int n = 0; n < ND; ++n)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c4 = 8 * n + 2 * j + g;  // float4 chunk of d = 32n + 8j + 4g
        const int phys = c4 ^ (l32 & (D / 4 - 1));
        const f32x4 val = {dq[n][4 * j], dq[n][4 * j + 1], dq[n][4 * j + 2], dq[n][4 * j + 3]};
        *(__attribute__((address_space(3))) f32x4 *)(part + (l32 * D + 4 * phys) * 4) = val;
      }
  }
  wait_lgkm0();
  barrier();
  // Output spans: a plain item writes the 128 dQ rows of its block (rows past c_q as 0),
  // a group item the 128 rows of each member block, member m's valid rows from wave m.
  const bool grouped = ROUTE == 128 && it.q < 0;
  const int n_spans = grouped ? NQG : 1;
  int32_t span_q[NQG], span_rows[NQG];
  if (grouped) {
    const FwdGroup &gr = a.fgroups[~it.q];
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
  constexpr int GROUPS = D / 8;
  for (int u = tid; u < n_spans * 128 * GROUPS; u += 64 * kDqWaves) {
    const int m = u / (128 * GROUPS), row = (u / GROUPS) & 127, grp = u % GROUPS;
    const int blk = span_q[m];
    if (blk < 0) continue;  // a group item without member m
    float acc8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (row < span_rows[m]) {
      const int qr = grouped ? row : row & 31, q_g = grouped ? m : row >> 5;
      for (int w = q_g; w < kDqWaves; w += NQG) {
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
    for (int e = 0; e < 8; ++e) out[e] = (__bf16)(acc8[e] * a.scale);
    const int64_t orow = bh * a.seq_q + 128 * blk + row;
    *(bf16x8 *)((char *)a.dq + (orow * D + 8 * grp) * 2) = out;
  }
}

// ---------------------------------------------------------------------------
// Owners split over several Q groups: sum their fp32 partials in group order (so the
// result does not depend on scheduling), scale dK, and write both by page id with the
// owner's row masks (rows past c_k as zeros, empty slots untouched).  HBM-bound: one
// workgroup per owner, 8 consecutive columns per thread.
template <int D>
__global__ __launch_bounds__(256) void kpage_bwd_kv_reduce(BwdArgs a) {
  constexpr int CH = D / 8;
  const BwdReduce r = a.reduce[blockIdx.x];
  const int32_t *own = a.owners + (int64_t)r.owner * 8;
  const uint32_t *kmk = a.owner_kmask + (int64_t)r.owner * 8;
  for (int e = threadIdx.x; e < 128 * CH; e += 256) {
    const int key = e / CH, c8 = (e % CH) * 8;
    const int slot = key >> 4, rin = key & 15;
    const uint32_t km = kmk[slot];
    if (km == 0u) continue;
    f32x4 sk0{}, sk1{}, sv0{}, sv1{};
    if ((km >> rin) & 1u) {
      for (int p = 0; p < r.count; ++p) {
        const float *pk = a.part + (int64_t)(r.part0 + p) * 2 * 128 * D + key * D + c8;
        const float *pv = pk + 128 * D;
        sk0 += *(const f32x4 *)pk;
        sk1 += *(const f32x4 *)(pk + 4);
        sv0 += *(const f32x4 *)pv;
        sv1 += *(const f32x4 *)(pv + 4);
      }
    }
    bf16x8 ok, ov;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ok[i] = (__bf16)(sk0[i] * a.scale);
      ok[4 + i] = (__bf16)(sk1[i] * a.scale);
      ov[i] = (__bf16)sv0[i];
      ov[4 + i] = (__bf16)sv1[i];
    }
    const int64_t row = (int64_t)r.bh * a.seq_kv + (int64_t)own[slot] * 16 + rin;
    *(bf16x8 *)((__bf16 *)a.dk + row * D + c8) = ok;
    *(bf16x8 *)((__bf16 *)a.dv + row * D + c8) = ov;
  }
}

// dQ over both routes in one launch, in the forward's launch order (order table: M128
// item i >= 0, else M64 or cleanup item ~i).  K half-tiles 0/1 and V half-tiles 0/1 in
// LDS; at the end the per-wave dQ partials.
template <int D>
__global__ __launch_bounds__(64 * kDqWaves, 2) void kpage_bwd_dq(BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[4 * 64 * D * 2];
  const int b = blockIdx.x;
  const int t = a.forder ? a.forder[b] : (b < a.n_fitems128 ? b : ~(b - a.n_fitems128));
  if (t >= 0) {
    if (a.froute_only != 64) dq_item<D, 128>(a, a.fitems128, t, smem);
  } else if (a.froute_only != 128) {
    dq_item<D, 64>(a, a.fitems64, ~t, smem);
  }
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs &a, hipStream_t stream, LaunchTimer *t) {
  if (a.max_uncovered > 0) {
    if (t) t->before(3, stream);
    hipLaunchKernelGGL(kpage_bwd_zero<D>, dim3((unsigned)(a.bh_count * a.max_uncovered)), dim3(256), 0, stream, a,
                       (int64_t)a.max_uncovered);
    if (t) t->after(3, stream);
  }
  if (t && t->split_routes()) {
    // profiling: the full dQ launch twice, one route's items each, at their positions in
    // the combined launch (the row statistics of both routes are written by the pair)
    BwdArgs only128 = a, only64 = a;
    only128.froute_only = 128;
    only64.froute_only = 64;
    const unsigned grid = (unsigned)(a.n_fitems128 + a.n_fitems64);
    if (grid > 0) {
      t->before(KPAGE_K_BWD_DQ, stream);
      hipLaunchKernelGGL(kpage_bwd_dq<D>, dim3(grid), dim3(64 * kDqWaves), 0, stream, only128);
      t->after(KPAGE_K_BWD_DQ, stream);
      t->before(KPAGE_K_BWD_DQ_Q64, stream);
      hipLaunchKernelGGL(kpage_bwd_dq<D>, dim3(grid), dim3(64 * kDqWaves), 0, stream, only64);
      t->after(KPAGE_K_BWD_DQ_Q64, stream);
    }
  } else if (a.n_fitems128 + a.n_fitems64 > 0) {
    if (t) t->before(KPAGE_K_BWD_DQ, stream);
    hipLaunchKernelGGL(kpage_bwd_dq<D>, dim3(a.n_fitems128 + a.n_fitems64), dim3(64 * kDqWaves), 0, stream, a);
    if (t) t->after(KPAGE_K_BWD_DQ, stream);
  }
  // the K/V-owned pass reads the lse2 and D that the dQ pass wrote
  if (a.n_items > 0) {
    if (t) t->before(4, stream);
    hipLaunchKernelGGL(kpage_bwd_kv<D>, dim3(a.n_items), dim3(64 * kKvWaves), 0, stream, a);
    if (t) t->after(4, stream);
  }
  if (a.n_reduce > 0) {
    if (t) t->before(6, stream);
    hipLaunchKernelGGL(kpage_bwd_kv_reduce<D>, dim3(a.n_reduce), dim3(256), 0, stream, a);
    if (t) t->after(6, stream);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs &a, int head_dim, hipStream_t stream, LaunchTimer *timer) {
  if (head_dim == 128) return launch_bwd_d<128>(a, stream, timer);
  if (head_dim == 64) return launch_bwd_d<64>(a, stream, timer);
  return hipErrorInvalidValue;
}

}  // namespace kpage
