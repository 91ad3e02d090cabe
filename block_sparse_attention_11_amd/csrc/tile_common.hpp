// Device helpers shared by the page-walking kernels (forward, backward dQ, backward
// dK/dV): LDS tile layouts, direct-to-LDS page copies, wait/barrier wrappers and
// compile-time loop helpers.  gfx950 (MI355X, CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <utility>

namespace kpage {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
// read-only tables indexed by wave-uniform values: the constant address space lets
// them go through scalar loads, which do not hold up the vector-memory counter
typedef const __attribute__((address_space(4))) int32_t c_i32;
typedef const __attribute__((address_space(4))) uint32_t c_u32;
typedef const __attribute__((address_space(4))) uint64_t c_u64;

constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;

// s_waitcnt immediates for gfx9: vmcnt[3:0] + vmcnt_hi[15:14], expcnt[6:4], lgkmcnt[11:8].
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// s_barrier alone.  It does not wait for the wave's own LDS or memory operations, and
// on gfx950 (which backs off barriers) the compiler inserts no wait before it either:
// a wave must wait (wait_lgkm0 / wait_vmcnt) for the LDS writes and reads that other
// waves depend on before calling it.
__device__ __forceinline__ void barrier() { __builtin_amdgcn_s_barrier(); }

template <int V>
struct ic {
  static constexpr int value = V;
};

template <int... I, class F>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, I...>, F &&f) {
  (f(ic<I>{}), ...);
}
// f(ic<0>{}), ..., f(ic<N-1>{}): every index is a compile-time constant.
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(std::make_integer_sequence<int, N>{}, f);
}

// Runs body(parity, flag, x) for x in [a, b), with parity = x & 1 as a compile-time
// value, so that LDS double buffers are addressed with constants.
template <class Flag, class Body>
__device__ __forceinline__ void for_range(Flag flag, int a, int b, Body &&body) {
  int x = a;
  if ((x & 1) && x < b) {
    body(ic<1>{}, flag, x);
    ++x;
  }
  for (; x + 1 < b; x += 2) {
    body(ic<0>{}, flag, x);
    body(ic<1>{}, flag, x + 1);
  }
  if (x < b) body(ic<0>{}, flag, x);
}

// ---- LDS tile layouts (row-major, 16-byte chunks XOR-swizzled per row) ----
//
// kSwzRow:  chunk ^ (row & (CH - 1)).  Row reads (ds_read_b128, one row per lane over
//           32 consecutive rows) are conflict-free.
// kSwzTr:   chunk ^ vswz(row): rows 4i..4i+3 get 0, 6, 12, 10.  A ds_read_b64_tr_b16
//           over 4 consecutive rows touches 8 (or 16) distinct chunk slots.
// kSwzBoth: chunk ^ swz(row): any 8 (or 16) aligned consecutive rows map one logical
//           chunk to distinct slots (row reads) and any 4 aligned consecutive rows map
//           a chunk pair to distinct slots (transposed reads), so one tile serves both.
enum Swizzle { kSwzRow = 0, kSwzTr = 1, kSwzBoth = 2 };

__host__ __device__ constexpr int vswz(int row) { return (0xAC60 >> (4 * (row & 3))) & 0xF; }
__host__ __device__ constexpr int swz(int r) {
  return (((0xAC60 >> (4 * (r & 3))) & 0xF) ^ ((r >> 2) & 1) ^ (((r >> 3) & 1) << 2));
}
template <int SWZ, int CH>
__host__ __device__ constexpr int swz_of(int row) {
  return (SWZ == kSwzRow ? row : SWZ == kSwzTr ? vswz(row) : swz(row)) & (CH - 1);
}

// Byte offset of logical 16-byte chunk `c` of row `row` in a tile of D-wide bf16 rows.
template <int SWZ, int D>
__device__ __forceinline__ int chunk_off(int row, int c) {
  return row * (D * 2) + ((c ^ swz_of<SWZ, D / 8>(row)) * 16);
}

// x ^ IMM as an opaque VALU op, so that the compiler recomputes per-access offsets
// next to their use instead of keeping one register per offset alive across a loop.
template <int IMM>
__device__ __forceinline__ int xor_imm(int x) {
  if constexpr (IMM == 0) {
    return x;
  } else {
    int r;
    asm volatile("v_xor_b32 %0, %1, %2" : "=v"(r) : "i"(IMM), "v"(x));
    return r;
  }
}

// Direct-to-LDS copy of SIZE (4 or 16) bytes per lane from sbase + voff to the LDS
// address `lds` + lane * SIZE (sbase and lds wave-uniform), written as inline assembly.
// The compiler's own waits for such copies cannot tell which LDS buffer a copy writes,
// so with the builtin it holds the first LDS read issued after a copy until that copy
// has landed, even when the read is of the other buffer of a double-buffered pair: the
// prefetch of the next step would then serialise with the current one.  Every caller
// orders copies and reads itself: wait_vmcnt, then a workgroup barrier, before a buffer
// written by copies is read.  M0 (the copy's LDS base) is an input operand of the asm,
// so the compiler writes it and knows it is in use; the s_nop covers the wait state
// between that write and the copy reading M0.
template <int SIZE>
__device__ __forceinline__ void lds_dma(const char *sbase, uint32_t voff, lds_char *lds) {
  static_assert(SIZE == 4 || SIZE == 16, "direct-to-LDS copies of 4 or 16 bytes per lane");
  const uint32_t m0 = (uint32_t)(uintptr_t)lds;
  if constexpr (SIZE == 16)
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "{m0}"(m0) : "memory");
  else
    asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1" : : "v"(voff), "s"(sbase), "{m0}"(m0) : "memory");
}

template <int SWZ, int CH>
constexpr bool swizzle_flip_is_uniform(int base, int n, int flip) {
  for (int r = 0; r < n; ++r)
    if ((swz_of<SWZ, CH>(base + r) ^ swz_of<SWZ, CH>(r)) != flip) return false;
  return true;
}

// One page (16 rows) of a bf16 [rows, D] tensor, global -> LDS rows r0 .. r0 + 15 of a
// tile (r0 % 16 == 0), 16 bytes per lane, laid out with swizzle SWZ.  `page` is
// wave-uniform, so the page base is a scalar address; each lane adds a 32-bit offset.
// Inside an aligned 16-row group every swizzle is linear in the row bits above the
// lane's own, so the offset of copy i is that of copy 0 with constant chunk bits
// flipped, plus i * ROWS_PER_INST rows.
template <int D, int SWZ>
__device__ __forceinline__ void load_page(const char *src, int32_t page, lds_char *tile, int r0, int lane) {
  constexpr int CH = D / 8;                    // 16-byte chunks per row
  constexpr int INSTS = 16 * CH / 64;          // direct loads per page
  constexpr int ROWS_PER_INST = 64 / CH;
  const char *pbase = src + (int64_t)page * (16 * D * 2);
  const int rin0 = lane / CH;
  const int off0 = rin0 * (D * 2) + (((lane % CH) ^ swz_of<SWZ, CH>(rin0)) * 16);
  static_for<INSTS>([&](auto i_c) __attribute__((always_inline)) {
    constexpr int I = decltype(i_c)::value;
    constexpr int FLIP = swz_of<SWZ, CH>(I * ROWS_PER_INST) ^ swz_of<SWZ, CH>(0);
    static_assert(swizzle_flip_is_uniform<SWZ, CH>(I * ROWS_PER_INST, ROWS_PER_INST, FLIP),
                  "swizzle must be linear in the copy index");
    // rows I * ROWS_PER_INST.. of the page: a scalar base, the lane offset unchanged
    // but for constant chunk bits
    const char *pi = pbase + I * ROWS_PER_INST * D * 2;
    asm volatile("" : "+s"(pi));  // keep the base scalar: saddr + 32-bit lane offset
    const uint32_t off = (uint32_t)xor_imm<16 * FLIP>(off0);
    lds_dma<16>(pi, off, (lds_char *)(tile + (r0 + I * ROWS_PER_INST) * D * 2));
  });
}

// Page `j` of tile `tile` of a page walk (one scalar load).
__device__ __forceinline__ int32_t tile_page(c_i32 *walk, int tile, int j) { return walk[8 * tile + j]; }

// Two transposed 4 x 16-bit reads (rows r0 and r0 + 8 of a 16-row group) joined into
// one MFMA operand of 8 bf16.
__device__ __forceinline__ bf16x8 tr_read8(const lds_char *p0, const lds_char *p1) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)p0);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)p1);
  const bf16x4 a = __builtin_bit_cast(bf16x4, lo), b = __builtin_bit_cast(bf16x4, hi);
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

__device__ __forceinline__ bf16x8 lds_read8(const lds_char *p) {
  return *(const __attribute__((address_space(3))) bf16x8 *)p;
}

// max(a, b, c) as one v_max3_f32.  Written out because the compiler otherwise
// canonicalises MFMA results (v_max x, x, x) before every fmaxf; the inputs here are
// scores and -inf, never signalling NaNs.
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Maximum of x over this lane and lane ^ 32 (v_permlane32_swap: a VALU op, no LDS).
__device__ __forceinline__ float half_max(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}

// x of this lane plus x of lane ^ 32 (the same sum, in the same order, in both lanes).
__device__ __forceinline__ float half_sum(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// Two floats to packed bf16 (round to nearest even), a in the low half: one
// v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// x, materialised here: an empty volatile asm keeps IR passes from sinking the
// computation of x past later control flow (the machine scheduler's fences do not
// bind them), so element-wise work stays in the MFMA slot it was written for.
__device__ __forceinline__ uint32_t pinned(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Key row (0..31) inside a 32 x 32 MFMA result block of accumulator register r in
// lane half g: rows 8 (r / 4) + 4 g + r % 4.
__device__ __forceinline__ constexpr int acc_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

// Lane mask (lanes 0..31: bit acc_row(R, 0) of `word`, lanes 32..63: bit acc_row(R, 1))
// for accumulator register R of a result block whose 32 rows have validity bits in the
// wave-uniform `word`: built with scalar operations.
template <int R>
__device__ __forceinline__ uint64_t row_lane_mask(uint32_t word) {
  const uint64_t lo = (word >> acc_row(R, 0)) & 1u, hi = (word >> acc_row(R, 1)) & 1u;
  return (lo * 0xFFFFFFFFull) | ((hi * 0xFFFFFFFFull) << 32);
}

// mask's bit of this lane ? x : y: one v_cndmask with the wave-uniform mask as its
// condition (from a select on a per-lane bit test the compiler emits three VALU ops).
// A builtin, not inline assembly, so that the compiler's wait-state checks cover the
// select's inputs (the same select written as inline assembly gave wrong results).
__device__ __forceinline__ float select_lanes(uint64_t mask, float x, float y) {
  return __builtin_amdgcn_inverse_ballot_w64(mask) ? x : y;
}

}  // namespace kpage
