// Internal helpers shared by the gfx950 kernels of libdsa (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// D = A * B + C on a 16x16 fp32 tile with a 32-deep bf16 contraction.  Lane l holds A row
// (l % 16) and B column (l % 16), 8 contraction values each for the lane group l / 16; the
// same (group, slot) pairs the same contraction index on both sides, so any consistent
// assignment of contraction indices to (group, slot) gives the exact dot product.  The
// result lane l, slot i is D[4 * (l / 16) + i][l % 16].
__device__ __forceinline__ f32x4 mfma16x16x32_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Same tile shape with a 128-deep OCP e4m3 contraction (32 bytes of A and B per lane,
// unit block scales).
__device__ __forceinline__ f32x4 mfma16x16x128_e4m3(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// LDS transpose read of four 16-bit values.  Within each group of 16 lanes, lane j reads
// 8 bytes at its own address; output lane i, element e is element (i % 4) of the 8 bytes
// read by lane 4 * e + i / 4.  Used to load an MFMA operand whose contraction index runs
// down the rows of a row-major LDS tile.
__device__ __forceinline__ i16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)((__attribute__((address_space(3))) char*)p));
}

// LDS access through address-space-3 pointers: in-bounds pointer arithmetic lets a base
// register plus a constant fold into the instruction's offset field (plain 32-bit integer
// addresses may wrap, so the compiler would add every constant in a register instead).
typedef __attribute__((address_space(3))) char lds_char;
typedef const lds_char* lds_ptr;

__device__ __forceinline__ lds_ptr lds_ptr_of(const void* p) {
  return (lds_ptr)(static_cast<const char*>(p));
}

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_ptr_of(p)));
}

__device__ __forceinline__ bf16x8 lds_load_bf16x8(lds_ptr p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(p);
}

__device__ __forceinline__ i16x4 lds_read_tr16_at(lds_ptr p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
}

__device__ __forceinline__ int64_t visible_pools(int64_t t, int64_t n_pools) {
  const int64_t v = (t + 1) >> 2;
  return v < n_pools ? (v < 0 ? 0 : v) : n_pools;
}

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (inputs are finite).
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

typedef float f32x8 __attribute__((ext_vector_type(8)));

// Splits eight fp32 values into bf16 operands hi + lo (hi = RNE(x), lo = RNE(x - hi)), so
// an MFMA over hi and lo sees x to about 16 significant bits.  Uses the hardware packed
// bf16 conversion.
__device__ __forceinline__ void split_bf16x8(f32x8 x, bf16x8& hi, bf16x8& lo) {
  hi = __builtin_convertvector(x, bf16x8);
  const f32x8 back = __builtin_convertvector(hi, f32x8);
  lo = __builtin_convertvector(x - back, bf16x8);
}

// Whole-vector reinterpretations between bf16 operands and their 16-bit patterns.
__device__ __forceinline__ bf16x8 bf16x8_from_bits(i16x8 bits) {
  return __builtin_bit_cast(bf16x8, bits);
}

__device__ __forceinline__ bf16x8 bf16x8_zero() {
  const i16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
  return bf16x8_from_bits(z);
}

// Order-preserving map of a float to uint32 (larger float -> larger key); -0 maps like +0.
__device__ __forceinline__ uint32_t float_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Cross-lane helpers (wave64).
__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }

}  // namespace dsa
