// Device-side helpers shared by the hyattn gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hy {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 16;  // tokens per KV block

// ---- bf16 <-> fp32 -----------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Round two floats to bf16, nearest-even (one v_cvt_pk_bf16_f32); the first
// lands in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

// Split a pair into hi + lo bf16 pairs: hi = RNE(x), lo = RNE(x - hi); hi + lo
// reproduces x to about 2^-17 relative.
__device__ __forceinline__ void split_bf16x2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16x2(x0, x1);
  lo = pack_bf16x2(x0 - bf16_lo(hi), x1 - bf16_hi(hi));
}

// ---- element I/O --------------------------------------------------------------
template <typename T> struct io;
template <> struct io<float> {
  static __device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void st(float* p, int64_t i, float x) { p[i] = x; }
};
template <> struct io<uint16_t> {
  static __device__ __forceinline__ float ld(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void st(uint16_t* p, int64_t i, float x) {
    p[i] = (uint16_t)f32_to_bf16_bits(x);
  }
};

// ---- MFMA -------------------------------------------------------------------
// v_mfma_f32_16x16x32_bf16: D(16x16) += A(16x32) * B(32x16).
// Lane l supplies row (l % 16) of A and column (l % 16) of B, eight k values
// each, with the same k positions in A and B; it receives rows
// 4 * (l / 16) + i (i = 0..3) of column l % 16 of D.
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// v_mfma_f32_32x32x16_bf16: D(32x32) += A(32x16) * B(16x32).
// Lane l supplies row (l % 32) of A and column (l % 32) of B, k values
// 8 * (l / 32) + e (e = 0..7) of each; it receives column l % 32 of D, rows
// 8 * (i / 4) + 4 * (l / 32) + (i % 4) in element i (i = 0..15). On gfx950 this
// shape sustains about twice the bf16 rate of 16x16x32 at one or two waves per
// SIMD (measured: 1.9-2.1 against 0.9-1.0 PFLOP/s), and the same rate at eight.
typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Row m = 8 g + 4 h + j (g = 0..3, h = 0..1, j = 0..3) of a 32-row operand of
// the product above taken to stand for index perm32(m) = 16 (g >> 1) + 8 h +
// 4 (g & 1) + j of the 32 indices it covers: a lane of half h (lanes 32 h ..
// 32 h + 31) then receives in accumulator element i the index
// 16 (i >> 3) + 8 h + (i & 7), i.e. eight consecutive indices per half-tile,
// which is a k operand of a following product (and a 16-byte bf16 piece).
__device__ __forceinline__ int perm32(int m) {
  const int g = m >> 3;
  return 16 * (g >> 1) + 8 * ((m >> 2) & 1) + 4 * (g & 1) + (m & 3);
}

// Transposing LDS read (ds_read_b64_tr_b16). Within each 16-lane group, lane
// i receives element i % 4 of the 8-byte chunks addressed by source lanes
// 4 j + i / 4 (j = 0..3) of its group. Hence if source lane s points at
// X[row0 + s / 4][c(s % 4)] of a row-major bf16 matrix X, lane i gets
// X[row0 + j][c(i / 4) + i % 4] for j = 0..3: four consecutive rows of one
// column, i.e. a k-contiguous MFMA operand read from a row-major tile.
// Issued as an opaque instruction: the compiler neither tracks it nor waits
// for it, so the caller must wait (lds_wait_all) before using the result. The
// compiler's own transposing-read intrinsic would drain every global-to-LDS
// load in flight before each read, which would serialise the kernels' rings.
__device__ __forceinline__ u32x2 ds_read_tr16_raw(const uint16_t* lds) {
  const uint32_t a = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const uint16_t*)lds));
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(a));
  return r;
}
// Wait until every outstanding LDS operation of the wave has completed; the
// registers passed in are tied to the wait so no use of them moves above it.
template <int N>
__device__ __forceinline__ void lds_wait_all(u32x4 (&x)[N]) {
  static_assert(N == 8 || N == 4 || N == 2 || N == 1, "lds_wait_all: 1, 2, 4 or 8 fragments");
  if constexpr (N == 8)
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]),
                   "+v"(x[6]), "+v"(x[7]));
  else if constexpr (N == 4)
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]));
  else if constexpr (N == 2)
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(x[0]), "+v"(x[1]));
  else
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(x[0]));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// acc + a.lo * b.lo + a.hi * b.hi for bf16 pairs, in fp32 (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b),
                                         acc, false);
}

// Workgroup barrier for LDS hand-offs only: waits for the wave's own LDS
// operations, then s_barrier. Unlike __syncthreads it has no release fence,
// so global stores and loads still in flight (outputs on their way to HBM,
// the next tile's prefetch) are not drained at every barrier. Only for
// kernels whose waves share data through LDS alone.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt untouched
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// s_waitcnt immediate that waits until at most n vector-memory operations are
// outstanding (expcnt and lgkmcnt left at their maxima): vmcnt is split over
// bits 3:0 and 15:14.
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

}  // namespace hy
