// Forward KPage attention for gfx950 (MI355X, CDNA4).
//
// KPage paper, section 3.2: every work item is one query block of one
// (batch, head).  Its K/V page walk is consumed one stage at a time: 8 Page16
// regions (128 key rows) for the M128 x N128 route, 16 (256 key rows) for the
// M64 x N256 route.  Each page is a contiguous 16-row run of the original K/V
// tensors and is copied straight from global memory into LDS with 16-byte
// direct-to-LDS loads (section 3.2.3); no compacted copy exists in HBM.  The
// consumer is an ordinary flash-attention step on the assembled tile: bf16
// MFMA for Q K^T and P V with fp32 accumulation, and an online softmax
// (section 3.2.4: invalid rows are set to -inf before the row maximum, and only
// on stages at or past the end of the fully valid prefix).
//
// Work split inside a 256-thread workgroup (4 waves of 64 lanes): each wave
// owns a 64-query x 64-key sub-tile of every stage.  M128: waves (w & 1) pick
// the query half and (w >> 1) the key half.  M64: all four waves share the 64
// query rows and take one key quarter each.  Every wave keeps its own running
// maximum, sum and output, and the waves are merged once at the end.
//
// Matrix layout per wave (v_mfma_f32_32x32x16_bf16):
//   S^T (key x query) = K . Q^T : A = K rows from LDS, B = Q rows kept in VGPRs.
//     A lane then holds 16 keys of one query column, so the row maximum is a
//     lane-local reduction plus one exchange with lane ^ 32.
//   O^T (dim x query) = V^T . P^T : B = the probabilities straight from the S^T
//     accumulators (same lane layout), A = V read transposed from LDS with
//     ds_read_b64_tr_b16.  The output column of a lane is again its own query,
//     so the per-query rescaling needs no cross-lane traffic.
#include <hip/hip_runtime.h>

#include "device.hpp"

namespace kpage {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
// read-only tables indexed by wave-uniform values: the constant address space lets
// them go through scalar loads, which do not hold up the vector-memory counter
typedef const __attribute__((address_space(4))) int32_t c_i32;
typedef const __attribute__((address_space(4))) uint32_t c_u32;

constexpr float kNegInf = -__builtin_inff();

// s_waitcnt immediates for gfx9: vmcnt[3:0] + vmcnt_hi[15:14], expcnt[6:4], lgkmcnt[11:8].
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
__device__ __forceinline__ void barrier() { __builtin_amdgcn_s_barrier(); }

// XOR swizzle of 16-byte chunks for V rows: rows 4i..4i+3 get 0, 6, 12, 10.  With
// it a ds_read_b64_tr_b16 over 4 consecutive rows touches 8 (or 16) distinct
// chunk slots, conflict-free for both 32- and 64-bank LDS.
__device__ __forceinline__ int vswz(int row) { return (0xAC60 >> (4 * (row & 3))) & 0xF; }

template <int D, int G>
__device__ __forceinline__ void load_stage(const char *kh, const char *vh, c_i32 *walk, lds_char *kb,
                                           lds_char *vb, int wave, int lane) {
  constexpr int CH = D / 8;                    // 16-byte chunks per row
  constexpr int PER_WAVE = G * 16 * CH / 256;  // direct loads per wave per tensor
  constexpr int ROWS_PER_INST = 64 / CH;
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int inst = wave * PER_WAVE + i;      // wave-uniform
    const int64_t page = walk[(inst * ROWS_PER_INST) >> 4];
    const int row = inst * ROWS_PER_INST + lane / CH;
    const int pos = lane % CH;
    const int64_t rbase = (page * 16 + (row & 15)) * (D * 2);
    const int ck = pos ^ (row & (CH - 1));
    const int cv = pos ^ (vswz(row) & (CH - 1));
    __builtin_amdgcn_global_load_lds((const void *)(kh + rbase + ck * 16), (lds_char *)(kb + inst * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((const void *)(vh + rbase + cv * 16), (lds_char *)(vb + inst * 1024), 16, 0, 0);
  }
}

template <int V>
struct ic {
  static constexpr int value = V;
};

template <int D, int G>
__global__ __launch_bounds__(256, 1) void kpage_fwd_kernel(FwdArgs args) {
  constexpr int CH = D / 8;          // 16-byte chunks per row
  constexpr int DS = D / 16;         // MFMA k-steps over the head dimension
  constexpr int ND = D / 32;         // 32-wide output blocks over the head dimension
  constexpr int M = G == 8 ? 128 : 64;
  constexpr int NBUF = G == 8 ? 2 : 1;
  constexpr int STAGE_BYTES = G * 16 * D * 2;

  __shared__ __attribute__((aligned(1024))) char kbuf0[STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char vbuf0[STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char kbuf1[NBUF == 2 ? STAGE_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) char vbuf1[NBUF == 2 ? STAGE_BYTES : 16];
  __shared__ float stat_m[4][64];
  __shared__ float stat_l[4][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int g = lane >> 5;           // lane half: selects 8 of the 16 k values of an MFMA operand
  const int l32 = lane & 31;

  const FwdItem it = args.items[blockIdx.x];
  const int bh = it.bh;
  const int cq = it.c_q;
  const int n_stages = it.walk_len / G;
  const int full_stages = it.n_full / G;
  const int qhalf = G == 8 ? (wave & 1) : 0;
  const int kvq = G == 8 ? (wave >> 1) : wave;
  const int kvbase = 64 * kvq;       // first key row of this wave inside a stage

  const char *kh = (const char *)args.k + (int64_t)bh * args.seq_kv * D * 2;
  const char *vh = (const char *)args.v + (int64_t)bh * args.seq_kv * D * 2;
  c_i32 *walk = (c_i32 *)(args.pages + it.walk_off);
  c_u32 *vwords = (c_u32 *)(args.valid + (it.walk_off >> 1));

  // per-wave fp32 partial output for the final merge, placed over the free stage buffers
  auto part_of = [&](int w) -> lds_char * {
    if (NBUF == 2)
      return w == 0 ? (lds_char *)kbuf0 : w == 1 ? (lds_char *)kbuf1 : w == 2 ? (lds_char *)vbuf0 : (lds_char *)vbuf1;
    return (w < 2 ? (lds_char *)kbuf0 : (lds_char *)vbuf0) + (w & 1) * (64 * D * 4);
  };

  if (n_stages > 0) load_stage<D, G>(kh, vh, walk, (lds_char *)kbuf0, (lds_char *)vbuf0, wave, lane);

  // Q rows of this wave as MFMA B operands: qreg[b][s] = Q[q0 + 32b + l32][16s + 8g .. +8]
  bf16x8 qreg[2][DS];
  {
    const int q0 = 128 * it.q + 64 * qhalf;
    const bf16x8 *qh = (const bf16x8 *)((const char *)args.q + ((int64_t)bh * args.seq_q + q0) * D * 2);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const bool ok = 64 * qhalf + 32 * b + l32 < cq;
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        bf16x8 x = qh[(32 * b + l32) * (D / 8) + 2 * s + g];
        if (!ok) x = bf16x8{};
        qreg[b][s] = x;
      }
    }
  }

  f32x16 oacc[ND][2];
#pragma unroll
  for (int n = 0; n < ND; ++n)
#pragma unroll
    for (int b = 0; b < 2; ++b) oacc[n][b] = f32x16{};
  float m_run[2] = {kNegInf, kNegInf};
  float l_run[2] = {0.f, 0.f};
  const float c2 = args.scale_log2;

  // lane-constant parts of the LDS addresses
  const int k_row_off = l32 * D * 2;
  const int k_swz = lane & (CH - 1) & 31;
  const int sl = lane & 15;
  const int mgrp = lane >> 4;
  const int v_row_off = (4 * g + (sl >> 2)) * D * 2;
  const int v_chunk_lane = 2 * (mgrp & 1) + ((sl & 3) >> 1);
  const int v_swz = vswz(sl >> 2) & (CH - 1);
  const int v_byte = (sl & 1) * 8;

  // One stage of the walk, reading LDS buffer BUF (a compile-time choice, so the
  // compiler can tell the prefetch into the other buffer apart from these reads).
  auto stage = [&](auto bufc, int st) {
    constexpr int BUF = decltype(bufc)::value;
    lds_char *kcur = BUF ? (lds_char *)kbuf1 : (lds_char *)kbuf0;
    lds_char *vcur = BUF ? (lds_char *)vbuf1 : (lds_char *)vbuf0;
    lds_char *knext = BUF ? (lds_char *)kbuf0 : (lds_char *)kbuf1;
    lds_char *vnext = BUF ? (lds_char *)vbuf0 : (lds_char *)vbuf1;
    if (NBUF == 1 && st > 0) load_stage<D, G>(kh, vh, walk + st * G, kcur, vcur, wave, lane);
    // validity words of this wave's two 32-key blocks (only read past the full prefix)
    uint32_t words[2] = {0xFFFFFFFFu, 0xFFFFFFFFu};
    const bool masked = st >= full_stages;
    if (masked) {
      words[0] = vwords[st * (G / 2) + 2 * kvq];
      words[1] = vwords[st * (G / 2) + 2 * kvq + 1];
    }
    wait_vmcnt<0>();
    wait_lgkm0();
    barrier();
    if (NBUF == 2 && st + 1 < n_stages) load_stage<D, G>(kh, vh, walk + (st + 1) * G, knext, vnext, wave, lane);
    const lds_char *kt = kcur + kvbase * D * 2;
    const lds_char *vt = vcur + kvbase * D * 2;

    // S^T = K Q^T for the wave's 64 keys x 64 queries
    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};
#pragma unroll
    for (int s = 0; s < DS; ++s) {
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const lds_char *src = kt + a * 32 * D * 2 + k_row_off + (((2 * s + g) ^ k_swz) * 16);
        const bf16x8 kop = *(const __attribute__((address_space(3))) bf16x8 *)src;
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qreg[b][s], acc[a][b], 0, 0, 0);
      }
    }

    // exact masking of invalid key rows on stages past the fully valid prefix
    if (masked) {
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const uint32_t word = words[a] >> (4 * g);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int bit = (r & 3) + 8 * ((r >> 2) & 1) + 16 * (r >> 3);
          if (!((word >> bit) & 1u)) {
            acc[a][0][r] = kNegInf;
            acc[a][1][r] = kNegInf;
          }
        }
      }
    }

    // online softmax per query column (lane-local over 32 keys, then lane ^ 32)
    bf16x8 pb[2][2][2];  // [a][b][hh]
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      float mx = kNegInf;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[a][b][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(m_run[b], mx);
      const float muse = mnew == kNegInf ? 0.f : mnew;
      const float alpha = __builtin_amdgcn_exp2f((m_run[b] - muse) * c2);
      m_run[b] = mnew;
      const float nm = -muse * c2;
      float rs = 0.f;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[a][b][8 * hh + e], c2, nm));
            rs += p;
            pb[a][b][hh][e] = (__bf16)p;
          }
      l_run[b] = l_run[b] * alpha + rs;
#pragma unroll
      for (int n = 0; n < ND; ++n) oacc[n][b] *= alpha;
    }

    // O^T += V^T P^T
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const lds_char *vrow = vt + (32 * a + 16 * hh) * D * 2 + v_row_off;
#pragma unroll
        for (int n = 0; n < ND; ++n) {
          const int chunk = ((4 * n + v_chunk_lane) ^ v_swz) * 16 + v_byte;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4 *)(vrow + chunk));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4 *)(vrow + 8 * D * 2 + chunk));
          const bf16x4 lo_b = __builtin_bit_cast(bf16x4, lo);
          const bf16x4 hi_b = __builtin_bit_cast(bf16x4, hi);
          const bf16x8 vop = {lo_b[0], lo_b[1], lo_b[2], lo_b[3], hi_b[0], hi_b[1], hi_b[2], hi_b[3]};
#pragma unroll
          for (int b = 0; b < 2; ++b)
            oacc[n][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb[a][b][hh], oacc[n][b], 0, 0, 0);
        }
      }
    if (NBUF == 1) {
      wait_lgkm0();
      barrier();
    }
  };

  if (NBUF == 2) {
    for (int st = 0; st < n_stages; st += 2) {
      stage(ic<0>{}, st);
      if (st + 1 < n_stages) stage(ic<1>{}, st + 1);
    }
  } else {
    for (int st = 0; st < n_stages; ++st) stage(ic<0>{}, st);
  }

  // ---- merge the waves that share query rows, then write O and LSE ----
  wait_vmcnt<0>();
  wait_lgkm0();
  barrier();
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const float lt = l_run[b] + __shfl_xor(l_run[b], 32);
    if (lane < 32) {
      stat_m[wave][32 * b + l32] = m_run[b];
      stat_l[wave][32 * b + l32] = lt;
    }
  }
  wait_lgkm0();
  barrier();
  lds_char *part = part_of(wave);
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int qr = 32 * b + l32;
    float mt = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const bool partner = G == 8 ? ((w & 1) == qhalf) : true;
      if (partner) mt = fmaxf(mt, stat_m[w][qr]);
    }
    float lt = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const bool partner = G == 8 ? ((w & 1) == qhalf) : true;
      if (partner && stat_m[w][qr] != kNegInf) lt += stat_l[w][qr] * __builtin_amdgcn_exp2f((stat_m[w][qr] - mt) * c2);
    }
    const float f = (m_run[b] == kNegInf || lt == 0.f) ? 0.f : __builtin_amdgcn_exp2f((m_run[b] - mt) * c2) / lt;
#pragma unroll
    for (int n = 0; n < ND; ++n) {
      f32x16 o = oacc[n][b] * f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c4 = 8 * n + 2 * j + g;                  // float4 chunk of d = 32n + 8j + 4g
        const int phys = c4 ^ (qr & (D / 4 - 1));
        const f32x4 val = {o[4 * j], o[4 * j + 1], o[4 * j + 2], o[4 * j + 3]};
        *(__attribute__((address_space(3))) f32x4 *)(part + (qr * D + 4 * phys) * 4) = val;
      }
    }
  }
  wait_lgkm0();
  barrier();

  const int64_t orow0 = (int64_t)bh * args.seq_q + 128 * it.q;
  const int vrows = cq < M ? cq : M;
  constexpr int GROUPS = D / 8;
  for (int u = tid; u < 128 * GROUPS; u += 256) {
    const int row = u / GROUPS, grp = u % GROUPS;
    float acc8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (row < vrows) {
      const int qr = row & 63;
      const int qh = row >> 6;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const bool partner = G == 8 ? ((w & 1) == qh) : true;
        if (!partner) continue;
        const lds_char *pw = part_of(w);
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
    *(bf16x8 *)((char *)args.o + ((orow0 + row) * D + 8 * grp) * 2) = out;
  }
  if (tid < 128) {
    const int row = tid;
    float lse = kNegInf;
    if (row < vrows) {
      const int qr = row & 63;
      const int qh = row >> 6;
      float mt = kNegInf;
      for (int w = 0; w < 4; ++w) {
        const bool partner = G == 8 ? ((w & 1) == qh) : true;
        if (partner) mt = fmaxf(mt, stat_m[w][qr]);
      }
      float lt = 0.f;
      for (int w = 0; w < 4; ++w) {
        const bool partner = G == 8 ? ((w & 1) == qh) : true;
        if (partner && stat_m[w][qr] != kNegInf) lt += stat_l[w][qr] * __builtin_amdgcn_exp2f((stat_m[w][qr] - mt) * c2);
      }
      if (mt != kNegInf && lt > 0.f) lse = mt * args.scale + __logf(lt);
    }
    args.lse[orow0 + row] = lse;
  }
}

}  // namespace

hipError_t launch_fwd(const FwdArgs &a, int head_dim, int route, hipStream_t stream, LaunchTimer *timer) {
  if (a.n_items <= 0) return hipSuccess;
  const int kid = route == 128 ? 0 : 1;
  dim3 grid(a.n_items), block(256);
  if (timer) timer->before(kid, stream);
  if (head_dim == 128 && route == 128) hipLaunchKernelGGL((kpage_fwd_kernel<128, 8>), grid, block, 0, stream, a);
  else if (head_dim == 128 && route == 64) hipLaunchKernelGGL((kpage_fwd_kernel<128, 16>), grid, block, 0, stream, a);
  else if (head_dim == 64 && route == 128) hipLaunchKernelGGL((kpage_fwd_kernel<64, 8>), grid, block, 0, stream, a);
  else if (head_dim == 64 && route == 64) hipLaunchKernelGGL((kpage_fwd_kernel<64, 16>), grid, block, 0, stream, a);
  else return hipErrorInvalidValue;
  if (timer) timer->after(kid, stream);
  return hipGetLastError();
}

}  // namespace kpage
