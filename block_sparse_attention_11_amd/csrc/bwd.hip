// Backward KPage attention for gfx950 (MI355X, CDNA4).
//
// KPage paper, section 3.3: the backward pass is organised around K/V owners.
// An owner is 8 Page16 slots (128 key rows) holding pages of one or more
// logical K/V blocks; no block crosses an owner.  Its reverse-Q neighbourhood
// is visited in steps of 8 query pages (128 query rows), and one 64-bit
// adjacency word per step (bit 8 j + i: Q slot j, K slot i) removes the page
// pairs that are not edges of the original graph (section 3.3.3).  dK and dV
// accumulate in registers over all steps of the owner; dQ goes through an fp32
// accumulator with atomic adds, scattered by query page id, and a final pass
// converts it to bf16 (section 3.3.3, last paragraph; section 3.4.1 for the
// cleanup of rows that hold no token).
//
// Kernels:
//   kpage_bwd_pre       D_i = sum_d dO_id O_id, LSE_i * log2(e) (0 for empty
//                       rows), zero the dQ accumulator.
//   kpage_bwd_zero      zero dK/dV pages that lie outside every block footprint.
//   kpage_bwd_main      one work item per (batch*head, owner).
//   kpage_bwd_post      dQ = bf16(scale * acc), rows past c_q set to 0.
//
// Main kernel layout (256 threads, 4 waves, v_mfma_f32_32x32x16_bf16): wave w
// owns key rows 32w..32w+31 of the owner (its K and V rows stay in VGPRs as MFMA
// operands, its dK and dV in accumulators).  Per step it computes, for all 128
// query rows, S = Q K^T with the lane index running over keys and the register
// index over queries; in that layout P^T and dS^T are directly the A operands
// of dV += P^T dO and dK += dS^T Q, whose B operands (columns of dO and Q) come
// from LDS through ds_read_b64_tr_b16.  dS is also written to LDS so that wave
// w can form dQ for query rows 32w..32w+31 over all 128 keys.
#include <hip/hip_runtime.h>
#include <hip/amd_detail/amd_hip_unsafe_atomics.h>

#include "device.hpp"

namespace kpage {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef const __attribute__((address_space(4))) int32_t c_i32;
typedef const __attribute__((address_space(4))) uint32_t c_u32;
typedef const __attribute__((address_space(4))) uint64_t c_u64;

constexpr float kLog2e = 1.4426950408889634f;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
__device__ __forceinline__ void barrier() { __builtin_amdgcn_s_barrier(); }

// XOR swizzle of the 16-byte chunks of row r of a row-major LDS tile.  Any 8
// (or 16) aligned consecutive rows map one logical chunk to 8 (16) distinct
// slots (row reads), and any 4 aligned consecutive rows map a chunk pair (quad)
// to 8 (16) distinct slots (ds_read_b64_tr_b16 reads): conflict-free for both
// access patterns on 32- and 64-bank LDS.
__device__ __forceinline__ int swz(int r) {
  return (((0xAC60 >> (4 * (r & 3))) & 0xF) ^ ((r >> 2) & 1) ^ (((r >> 3) & 1) << 2));
}

__device__ __forceinline__ bf16x8 tr_read8(const lds_char *p0, const lds_char *p1) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)p0);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)p1);
  const bf16x4 a = __builtin_bit_cast(bf16x4, lo), b = __builtin_bit_cast(bf16x4, hi);
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// ---------------------------------------------------------------------------
// pre: 16 threads per query row
template <int D>
__global__ __launch_bounds__(256) void kpage_bwd_pre(BwdArgs a) {
  const int64_t rows = (int64_t)a.bh_count * a.seq_q;
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  if (row >= rows) return;
  constexpr int PER = D / 16;  // elements per thread
  const __bf16 *o = (const __bf16 *)a.o + row * D + sub * PER;
  const __bf16 *g = (const __bf16 *)a.dout + row * D + sub * PER;
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) s += (float)o[e] * (float)g[e];
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) s += __shfl_xor(s, off, 16);
  float *acc = a.dq_acc + row * D + sub * PER;
#pragma unroll
  for (int e = 0; e < PER; e += 4) *(f32x4 *)(acc + e) = f32x4{0.f, 0.f, 0.f, 0.f};
  if (sub == 0) {
    a.delta[row] = s;
    const float l = a.lse[row];
    a.delta[rows + row] = l == -__builtin_inff() ? 0.f : l * kLog2e;
  }
}

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

// post: 16 threads per query row
template <int D>
__global__ __launch_bounds__(256) void kpage_bwd_post(BwdArgs a) {
  const int64_t rows = (int64_t)a.bh_count * a.seq_q;
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  if (row >= rows) return;
  constexpr int PER = D / 16;
  const int64_t bh = row / a.seq_q;
  const int64_t r = row % a.seq_q;
  const int slot = a.per_head ? (int)bh : 0;
  const bool valid = (r & 127) < a.q_valid[(int64_t)slot * a.n_q + (r >> 7)];
  const float *acc = a.dq_acc + row * D + sub * PER;
  __bf16 *out = (__bf16 *)a.dq + row * D + sub * PER;
  typedef __bf16 row_t __attribute__((ext_vector_type(PER)));
  row_t v;
#pragma unroll
  for (int j = 0; j < PER; ++j) v[j] = (__bf16)(valid ? acc[j] * a.scale : 0.f);
  *(row_t *)out = v;
}

// ---------------------------------------------------------------------------
// main

template <int D>
__device__ __forceinline__ void load_qstep(const char *qh, const char *gh, const float *lse2h, const float *delh,
                                           c_i32 *qp, lds_char *qb, lds_char *gb, lds_char *lb, lds_char *db,
                                           int wave, int lane) {
  constexpr int CH = D / 8;
  constexpr int PER_WAVE = 128 * CH / 256;  // 16-byte direct loads per wave per tensor
  constexpr int ROWS_PER_INST = 64 / CH;
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int inst = wave * PER_WAVE + i;
    const int64_t page = qp[(inst * ROWS_PER_INST) >> 4];
    const int row = inst * ROWS_PER_INST + lane / CH;
    const int pos = lane % CH;
    const int c = pos ^ (swz(row) & (CH - 1));
    const int64_t off = (page * 16 + (row & 15)) * (D * 2) + c * 16;
    __builtin_amdgcn_global_load_lds((const void *)(qh + off), (lds_char *)(qb + inst * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((const void *)(gh + off), (lds_char *)(gb + inst * 1024), 16, 0, 0);
  }
  // LSE * log2(e) and D of the 128 rows: one 4-byte direct load per lane, waves 0-1 and 2-3
  {
    const int half = wave & 1;
    const int row = 64 * half + lane;
    // the 4 pages of this half as scalar loads, then a per-lane pick
    const int64_t p0 = qp[4 * half], p1 = qp[4 * half + 1], p2 = qp[4 * half + 2], p3 = qp[4 * half + 3];
    const int sel = lane >> 4;
    const int64_t page = sel == 0 ? p0 : sel == 1 ? p1 : sel == 2 ? p2 : p3;
    const float *src = (wave < 2 ? lse2h : delh) + page * 16 + (row & 15);
    lds_char *dst = (wave < 2 ? lb : db) + half * 256;
    __builtin_amdgcn_global_load_lds((const void *)src, (lds_char *)dst, 4, 0, 0);
  }
}

template <int D>
__global__ __launch_bounds__(256, 1) void kpage_bwd_main(BwdArgs a) {
  constexpr int CH = D / 8;
  constexpr int DS = D / 16;  // k-steps over the head dimension
  constexpr int ND = D / 32;  // 32-wide output blocks over the head dimension
  constexpr int TILE = 128 * D * 2;

  __shared__ __attribute__((aligned(1024))) char k_lds[TILE];
  __shared__ __attribute__((aligned(1024))) char q_lds[TILE];
  __shared__ __attribute__((aligned(1024))) char g_lds[TILE];
  __shared__ __attribute__((aligned(1024))) char s_lds[128 * 128 * 2];
  __shared__ __attribute__((aligned(256))) float lse_lds[128];
  __shared__ __attribute__((aligned(256))) float del_lds[128];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int sl = lane & 15;
  const int mgrp = lane >> 4;

  const BwdItem it = a.items[blockIdx.x];
  const int64_t bh = it.bh;
  const int n_steps = it.n_steps;
  c_i32 *own = (c_i32 *)(a.owners + (int64_t)it.owner * 8);
  c_u32 *kmk = (c_u32 *)(a.owner_kmask + (int64_t)it.owner * 8);
  c_i32 *qpages = (c_i32 *)(a.qpages + it.qwalk_off);
  c_u32 *qmasks = (c_u32 *)(a.qmask + it.qwalk_off);
  c_u64 *adjw = (c_u64 *)(a.adj + (it.qwalk_off >> 3));

  const char *kh = (const char *)a.k + bh * a.seq_kv * D * 2;
  const char *vh = (const char *)a.v + bh * a.seq_kv * D * 2;
  const char *qh = (const char *)a.q + bh * a.seq_q * D * 2;
  const char *gh = (const char *)a.dout + bh * a.seq_q * D * 2;
  const int64_t rows_all = (int64_t)a.bh_count * a.seq_q;
  const float *delh = a.delta + bh * a.seq_q;
  const float *lse2h = a.delta + rows_all + bh * a.seq_q;
  float *dqh = a.dq_acc + bh * a.seq_q * D;

  // owner slots: empty slots read the first page (finite data) and are masked out
  int32_t opage[8];
  uint32_t okm[8];
  bool all_k = true;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    okm[i] = kmk[i];
    opage[i] = own[i] >= 0 ? own[i] : own[0];
    all_k = all_k && okm[i] == 0xFFFFu;
  }

  // owner K into LDS (for dQ), rows = slot * 16 + r
  {
    constexpr int PER_WAVE = 128 * CH / 256;
    constexpr int ROWS_PER_INST = 64 / CH;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int inst = wave * PER_WAVE + i;
      const int slot = (inst * ROWS_PER_INST) >> 4;
      int64_t page = opage[0];
#pragma unroll
      for (int j = 1; j < 8; ++j)
        if (slot == j) page = opage[j];
      const int row = inst * ROWS_PER_INST + lane / CH;
      const int c = (lane % CH) ^ (swz(row) & (CH - 1));
      __builtin_amdgcn_global_load_lds((const void *)(kh + (page * 16 + (row & 15)) * (D * 2) + c * 16),
                                       (lds_char *)((lds_char *)k_lds + inst * 1024), 16, 0, 0);
    }
  }
  if (n_steps > 0)
    load_qstep<D>(qh, gh, lse2h, delh, qpages, (lds_char *)q_lds, (lds_char *)g_lds, (lds_char *)lse_lds,
                  (lds_char *)del_lds, wave, lane);

  // this wave's 32 key rows as MFMA B operands (k = head dim, j = key)
  const int kslot = 2 * wave + (l32 >> 4);
  int64_t mypage = opage[0];
  uint32_t mykm = okm[0];
#pragma unroll
  for (int j = 1; j < 8; ++j)
    if (kslot == j) {
      mypage = opage[j];
      mykm = okm[j];
    }
  const bool kvalid = (mykm >> (l32 & 15)) & 1u;
  bf16x8 kreg[DS], vreg[DS];
  {
    const bf16x8 *kr = (const bf16x8 *)(kh + (mypage * 16 + (l32 & 15)) * (D * 2));
    const bf16x8 *vr = (const bf16x8 *)(vh + (mypage * 16 + (l32 & 15)) * (D * 2));
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      kreg[s] = kr[2 * s + g];
      vreg[s] = vr[2 * s + g];
    }
  }

  f32x16 dk[ND], dv[ND];
#pragma unroll
  for (int n = 0; n < ND; ++n) {
    dk[n] = f32x16{};
    dv[n] = f32x16{};
  }
  const float c2 = a.scale_log2;

  // lane-constant parts of LDS addresses
  const int row_rd = l32;                                   // row reads: row = 32 qb + l32
  const int tr_row = 4 * g + (sl >> 2);                     // tr reads: row offset inside 16 rows
  const int tr_col = 2 * (mgrp & 1) + ((sl & 3) >> 1);      // tr reads: chunk inside 4 chunks
  const int tr_byte = (sl & 1) * 8;

  for (int st = 0; st < n_steps; ++st) {
    wait_vmcnt<0>();
    wait_lgkm0();
    barrier();
    // per-step masks: adjacency word and row masks of the 8 query pages
    const uint64_t adj = adjw[st];
    uint32_t qm[8];
    bool all_q = true;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      qm[j] = qmasks[8 * st + j];
      all_q = all_q && qm[j] == 0xFFFFu;
    }
    const bool all_valid = all_q && all_k && adj == ~0ull;
    // per query page: rows of this lane's half (shifted by 4g) that pair with this lane's key
    uint32_t pm[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      pm[j] = (kvalid && ((adj >> (8 * j + kslot)) & 1ull)) ? (qm[j] >> (4 * g)) : 0u;

#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      // S = Q K^T and dP = dO V^T for query rows 32qb..32qb+31 (lane = key)
      f32x16 s_acc = f32x16{}, dp_acc = f32x16{};
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        const int r = 32 * qb + row_rd;
        const int off = r * (D * 2) + (((2 * s + g) ^ (swz(r) & (CH - 1))) * 16);
        const bf16x8 qop = *(const __attribute__((address_space(3))) bf16x8 *)((lds_char *)q_lds + off);
        const bf16x8 gop = *(const __attribute__((address_space(3))) bf16x8 *)((lds_char *)g_lds + off);
        s_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qop, kreg[s], s_acc, 0, 0, 0);
        dp_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(gop, vreg[s], dp_acc, 0, 0, 0);
      }
      // P = exp(scale S - LSE) on valid pairs, dS = P (dP - D)
      bf16x8 pb[2], sb[2];
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const int q0 = 32 * qb + 8 * j4 + 4 * g;
        const f32x4 l4 = *(const __attribute__((address_space(3))) f32x4 *)((lds_char *)lse_lds + q0 * 4);
        const f32x4 d4 = *(const __attribute__((address_space(3))) f32x4 *)((lds_char *)del_lds + q0 * 4);
        const int page = 2 * qb + (j4 >> 1);
        const uint32_t bits = pm[page] >> (8 * (j4 & 1));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * j4 + e;
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s_acc[r], c2, -l4[e]));
          if (!all_valid && !((bits >> e) & 1u)) p = 0.f;
          const float ds = p * (dp_acc[r] - d4[e]);
          pb[r >> 3][r & 7] = (__bf16)p;
          sb[r >> 3][r & 7] = (__bf16)ds;
        }
      }
      // dS to LDS for dQ: row = key (32w + l32), columns = query rows
      {
        const int kr = 32 * wave + l32;
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
          const int chunk = (4 * qb + j4) ^ swz(kr);
          const bf16x4 v = {sb[j4 >> 1][4 * (j4 & 1)], sb[j4 >> 1][4 * (j4 & 1) + 1], sb[j4 >> 1][4 * (j4 & 1) + 2],
                            sb[j4 >> 1][4 * (j4 & 1) + 3]};
          *(__attribute__((address_space(3))) bf16x4 *)((lds_char *)s_lds + kr * 256 + chunk * 16 + g * 8) = v;
        }
      }
      // dV += P^T dO and dK += dS^T Q over these 32 query rows
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int rbase = 32 * qb + 16 * hh + tr_row;
#pragma unroll
        for (int n = 0; n < ND; ++n) {
          const int r0 = rbase, r1 = rbase + 8;
          const int c0 = ((4 * n + tr_col) ^ (swz(r0) & (CH - 1))) * 16 + tr_byte;
          const int c1 = ((4 * n + tr_col) ^ (swz(r1) & (CH - 1))) * 16 + tr_byte;
          const bf16x8 gop = tr_read8((lds_char *)g_lds + r0 * (D * 2) + c0, (lds_char *)g_lds + r1 * (D * 2) + c1);
          const bf16x8 qop = tr_read8((lds_char *)q_lds + r0 * (D * 2) + c0, (lds_char *)q_lds + r1 * (D * 2) + c1);
          dv[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pb[hh], gop, dv[n], 0, 0, 0);
          dk[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sb[hh], qop, dk[n], 0, 0, 0);
        }
      }
    }
    wait_lgkm0();
    barrier();
    if (st + 1 < n_steps)
      load_qstep<D>(qh, gh, lse2h, delh, qpages + 8 * (st + 1), (lds_char *)q_lds, (lds_char *)g_lds,
                    (lds_char *)lse_lds, (lds_char *)del_lds, wave, lane);

    // dQ for query rows 32w..32w+31: A = dS (tr reads of the key-major dS tile), B = K (tr reads)
    f32x16 dq[ND];
#pragma unroll
    for (int n = 0; n < ND; ++n) dq[n] = f32x16{};
#pragma unroll
    for (int ka = 0; ka < 4; ++ka)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int r0 = 32 * ka + 16 * hh + tr_row, r1 = r0 + 8;
        const int sc0 = ((4 * wave + tr_col) ^ swz(r0)) * 16 + tr_byte;
        const int sc1 = ((4 * wave + tr_col) ^ swz(r1)) * 16 + tr_byte;
        const bf16x8 sop = tr_read8((lds_char *)s_lds + r0 * 256 + sc0, (lds_char *)s_lds + r1 * 256 + sc1);
#pragma unroll
        for (int n = 0; n < ND; ++n) {
          const int c0 = ((4 * n + tr_col) ^ (swz(r0) & (CH - 1))) * 16 + tr_byte;
          const int c1 = ((4 * n + tr_col) ^ (swz(r1) & (CH - 1))) * 16 + tr_byte;
          const bf16x8 kop = tr_read8((lds_char *)k_lds + r0 * (D * 2) + c0, (lds_char *)k_lds + r1 * (D * 2) + c1);
          dq[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sop, kop, dq[n], 0, 0, 0);
        }
      }
    // scatter-add into the fp32 accumulator by query page (rows without a token are skipped)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int j = 2 * wave + half;
      const uint32_t rows = qm[j] >> (4 * g);
      float *dst = dqh + ((int64_t)qpages[8 * st + j] * 16 + 4 * g) * D + l32;
#pragma unroll
      for (int r8 = 0; r8 < 8; ++r8) {
        const int r = 8 * half + r8;
        const int rin = 8 * ((r8 >> 2) & 1) + (r8 & 3);  // row inside the page minus 4g
        if ((rows >> rin) & 1u) {
#pragma unroll
          for (int n = 0; n < ND; ++n) unsafeAtomicAdd(dst + rin * D + 32 * n, dq[n][r]);
        }
      }
    }
  }

  wait_vmcnt<0>();
  // dK (scaled) and dV to their pages; rows past the block's valid count and empty slots handled
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int key = 32 * wave + 8 * (r >> 2) + 4 * g + (r & 3);
    const int slot = key >> 4;
    const int rin = key & 15;
    uint32_t km = okm[0];
    int64_t page = opage[0];
#pragma unroll
    for (int j = 1; j < 8; ++j)
      if (slot == j) {
        km = okm[j];
        page = opage[j];
      }
    if (km == 0u) continue;  // empty owner slot
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

template <int D>
hipError_t launch_bwd_d(const BwdArgs &a, hipStream_t stream, LaunchTimer *t) {
  const int64_t rows = (int64_t)a.bh_count * a.seq_q;
  const int64_t row_blocks = (rows + 15) / 16;
  if (t) t->before(2, stream);
  hipLaunchKernelGGL(kpage_bwd_pre<D>, dim3((unsigned)row_blocks), dim3(256), 0, stream, a);
  if (t) t->after(2, stream);
  if (a.max_uncovered > 0) {
    if (t) t->before(3, stream);
    hipLaunchKernelGGL(kpage_bwd_zero<D>, dim3((unsigned)(a.bh_count * a.max_uncovered)), dim3(256), 0, stream, a,
                       (int64_t)a.max_uncovered);
    if (t) t->after(3, stream);
  }
  if (a.n_items > 0) {
    if (t) t->before(4, stream);
    hipLaunchKernelGGL(kpage_bwd_main<D>, dim3(a.n_items), dim3(256), 0, stream, a);
    if (t) t->after(4, stream);
  }
  if (t) t->before(5, stream);
  hipLaunchKernelGGL(kpage_bwd_post<D>, dim3((unsigned)row_blocks), dim3(256), 0, stream, a);
  if (t) t->after(5, stream);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs &a, int head_dim, hipStream_t stream, LaunchTimer *timer) {
  if (head_dim == 128) return launch_bwd_d<128>(a, stream, timer);
  if (head_dim == 64) return launch_bwd_d<64>(a, stream, timer);
  return hipErrorInvalidValue;
}

}  // namespace kpage
