// Device-side helpers shared by the gfx950 kernels of the linear-attention
// library: vector types, the bf16 matrix-core instruction, the transposing
// LDS read, and bf16 packing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lal {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16;

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16).
// Operand layouts (lane l, g = l / 16, slot e):
//   A: row l%16, K index 8g+e;  B: column l%16, K index 8g+e;
//   D: column l%16, rows 4g+e (e < 4).
// Only the pairing of A and B slots matters for the K index, so both operands
// may use any common relabelling of K.
__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Transposing 8-byte LDS read (ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane i receives in slot e the (i % 4)-th 16-bit element of the
// 8 bytes addressed by lane 4e + i/4 of the same group.  With lane t of the
// group addressing row R0 + t/4, columns C0 + 4(t%4) .. +3 of a row-major
// 16-bit tile, lane i therefore receives column C0 + i, rows R0 .. R0+3.
__device__ __forceinline__ s16x4 lds_read_tr(const u16 *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4 *)((__attribute__((address_space(3))) u16 *)(p)));
}

__device__ __forceinline__ bf16x8 join_tr(s16x4 lo, s16x4 hi) {
  s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Round four fp32 values to bf16 (nearest even) and pack them into 8 bytes.
__device__ __forceinline__ uint2 pack_bf16x4(f32x4 x) {
  bf16x4 b = {(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
  return __builtin_bit_cast(uint2, b);
}

// Buffer resource for raw buffer loads over `bytes` bytes from `base`
// (stride 0, 32-bit data format); accesses at or past `bytes` return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ float bf16_bits_to_f32(u16 b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

__device__ __forceinline__ u16 f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(u16, (bf16)x);
}

// OCP FP8 E4M3 ("e4m3fn": 1 sign bit, 4 exponent bits with bias 7, 3
// fraction bits, no infinity, largest finite 448) through gfx950's
// converters, which round to nearest even.  The converter turns values past
// the largest finite one into NaN, so finite values are clamped to +-448
// first (NaN and infinities then store +-448 too).
__device__ __forceinline__ uint32_t f32_to_e4m3x4(f32x4 x) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(x[0], -448.f, 448.f),
                                          __builtin_amdgcn_fmed3f(x[1], -448.f, 448.f), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(x[2], -448.f, 448.f),
                                      __builtin_amdgcn_fmed3f(x[3], -448.f, 448.f), w, true);
  return (uint32_t)w;  // byte e holds x[e]
}

// The four codes of a 32-bit word (byte 0 first), widened exactly to fp32.
__device__ __forceinline__ f32x4 e4m3x4_to_f32(uint32_t w) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  return f32x4{lo[0], lo[1], hi[0], hi[1]};
}

}  // namespace lal
