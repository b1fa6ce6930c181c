// Device-side building blocks for the gfx950 (CDNA4) kernels: bf16 packing,
// DPP lane exchanges, LDS DMA issue and wait, exp2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// LDS scratch is written and read back at different widths (bf16 weights
// stored singly, read in pairs); these types keep type-based alias analysis
// from reordering such accesses.
typedef uint16_t __attribute__((may_alias)) u16_alias;
typedef uint32_t __attribute__((may_alias)) u32_alias;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// v_dot2c_f32_bf16: a.x*b.x + a.y*b.y + c, products exact in fp32.
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

// Two fp32 -> packed bf16 (lo = a, hi = b), round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  f32x2 f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __builtin_bit_cast(float, x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) {
  return __builtin_bit_cast(float, x & 0xffff0000u);
}

// Byte permutes selecting the low (resp. high) bf16 halves of two dwords:
// lo_pair(x, y) = (x.lo, y.lo), hi_pair(x, y) = (x.hi, y.hi).
__device__ __forceinline__ uint32_t lo_pair(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x05040100u);
}
__device__ __forceinline__ uint32_t hi_pair(uint32_t x, uint32_t y) {
  return __builtin_amdgcn_perm(y, x, 0x07060302u);
}

// DPP lane exchange of a float.  Controls used: quad_perm [1,0,3,2] (0xB1),
// quad_perm [2,3,0,1] (0x4E), row_ror:4 (0x124), row_ror:8 (0x128).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               0xF, 0xF, false));
}

// Matrix-core products on 16x16 fp32 tiles (wave64 operand layouts, lane l):
//   A[row = l % 16][k = K/4 * (l / 16) + e], B[k = K/4 * (l / 16) + e][col = l % 16],
//   C/D[row = 4 * (l / 16) + i][col = l % 16], e < K/4, i < 4.
// mfma_k32: v_mfma_f32_16x16x32_bf16 (8 bf16 of A and of B per lane).
__device__ __forceinline__ f32x4 mfma_k32(const uint4 &a, const uint4 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// mfma_k16: v_mfma_f32_16x16x16_bf16 (4 bf16 of A and of B per lane).
__device__ __forceinline__ f32x4 mfma_k16(const uint2 &a, const uint2 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                   __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// ds_read_b64_tr_b16: each lane names 8 bytes (4 bf16) of LDS; within every
// group of 16 lanes, lane i receives as element j (j < 4) element i % 4 of
// the 8 bytes named by lane 4 j + i / 4.  Reading 4 rows x 16 columns of a
// row-major bf16 tile this way hands lane i column i of those 4 rows.
__device__ __forceinline__ uint2 read_tr(const char *p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4 *)(__attribute__((address_space(3))) void *)p);
  return __builtin_bit_cast(uint2, v);
}

typedef int i32x2 __attribute__((ext_vector_type(2)));

// ds_read_b64_tr_b8: within each group of 16 lanes, lane c receives as its
// byte k (k < 8) byte c % 8 of the 8 bytes addressed by lane 2 k + c / 8 of
// its group: the 8 rows addressed by lane pairs, column c.
__device__ __forceinline__ uint2 read_tr8(const char *p) {
  const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) i32x2 *)(__attribute__((address_space(3))) void *)p);
  return __builtin_bit_cast(uint2, v);
}

// ---- fp8 (OCP e4m3) codes ----
// 4 codes -> 4 bf16 values (exact: every e4m3 value is a bf16 value), element
// order kept.
__device__ __forceinline__ uint2 fp8x4_to_bf16(uint32_t v) {
  return uint2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.f, true))};
}
// 8 codes -> 8 bf16 values, element order kept.
__device__ __forceinline__ uint4 fp8x8_to_bf16(uint2 v) {
  return uint4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.f, true)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.f, true))};
}

__device__ __forceinline__ float clamp448(float y) {
  return y > 448.f ? 448.f : (y < -448.f ? -448.f : y);
}

// 8 bf16 values -> their 8 codes: e4m3 of clamp(x * inv, -448, 448), the
// product in fp32, rounded to nearest even; the comparisons keep a NaN
// product NaN.
__device__ __forceinline__ uint2 quantize8(uint4 x, float inv) {
  auto lo = [&](uint32_t w) { return clamp448(__uint_as_float(w << 16) * inv); };
  auto hi = [&](uint32_t w) { return clamp448(__uint_as_float(w & 0xFFFF0000u) * inv); };
  // word_sel false fills bytes 0-1, true bytes 2-3 (keeping the others)
  int a = __builtin_amdgcn_cvt_pk_fp8_f32(lo(x.x), hi(x.x), 0, false);
  a = __builtin_amdgcn_cvt_pk_fp8_f32(lo(x.y), hi(x.y), a, true);
  int b = __builtin_amdgcn_cvt_pk_fp8_f32(lo(x.z), hi(x.z), 0, false);
  b = __builtin_amdgcn_cvt_pk_fp8_f32(lo(x.w), hi(x.w), b, true);
  return uint2{(uint32_t)a, (uint32_t)b};
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Max of x over the 64 lanes of the wave, returned in every lane.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x124>(x));
  x = fmaxf(x, dpp<0x128>(x));
  float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
  float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16));
  float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
  float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Max over lanes that differ only in bits 2..5 (the 16 "token" lanes of a
// 4-lanes-per-token layout); lanes of one quad already agree.
__device__ __forceinline__ float max_over_quads(float x) {
  x = fmaxf(x, dpp<0x124>(x));
  x = fmaxf(x, dpp<0x128>(x));
  float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
  float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16));
  float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
  float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Sum over lanes that differ only in bits 2..5, in every lane.
__device__ __forceinline__ float sum_over_quads(float x) {
  x += dpp<0x124>(x);
  x += dpp<0x128>(x);
  float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
  float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16));
  float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
  float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48));
  return (r0 + r1) + (r2 + r3);
}

// Sum of x over the 64 lanes of the wave, returned in every lane.
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  return sum_over_quads(x);
}

// Sum of the 4 lanes of each quad, in every lane of the quad.
__device__ __forceinline__ float quad_sum(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  return x;
}

// Read-only view in the constant address space: a wave-uniform index then
// compiles to a scalar (SMEM) load, counted by lgkmcnt rather than vmcnt, so it
// never waits behind LDS DMA traffic.
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(4))) T *as_const(const T *p) {
  return (const __attribute__((address_space(4))) T *)(p);
}

// LDS byte offset of a __shared__ pointer.
template <typename T>
__device__ __forceinline__ uint32_t lds_offset(T *p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) void *)p);
}

// One wave-wide 16-byte-per-lane DMA from global memory into LDS
// (global_load_lds_dwordx4): lane i reads 16 bytes at base + voff and writes
// them to LDS bytes [lds + 16 i, lds + 16 i + 16).  `lds` and `base` must be
// wave-uniform.  The load is counted by vmcnt; the caller waits with
// wait_vmcnt before reading the LDS bytes.  Outstanding LDS reads are drained
// first (lgkmcnt(0)) so a buffer is never overwritten under a pending read.
// M0 is saved and restored around the use.
__device__ __forceinline__ void dma16(uint32_t lds, const void *base, uint32_t voff) {
  // Both are wave-uniform by contract; readfirstlane puts them in SGPRs even
  // where the compiler cannot prove uniformity.
  lds = __builtin_amdgcn_readfirstlane(lds);
  const uint64_t b64 = (uint64_t)(uintptr_t)base;
  base = (const void *)(uintptr_t)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b64 >> 32))
                                    << 32) |
                                   (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b64));
  uint32_t saved;
  asm volatile(
      "s_waitcnt lgkmcnt(0)\n\t"
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(base)
      : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Runtime-count wait: the count is one of a few compile-time values.
template <int STEP, int MAXK>
__device__ __forceinline__ void wait_vmcnt_steps(int k) {
  if constexpr (MAXK >= 3) {
    if (k >= 3) { wait_vmcnt<3 * STEP>(); return; }
  }
  if constexpr (MAXK >= 2) {
    if (k == 2) { wait_vmcnt<2 * STEP>(); return; }
  }
  if constexpr (MAXK >= 1) {
    if (k == 1) { wait_vmcnt<STEP>(); return; }
  }
  wait_vmcnt<0>();
}

}  // namespace pa
