// Device helpers shared by the libkda kernels: storage conversions, MFMA operand types
// and the lane layout of the gfx950 16x16x32 matrix instructions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;

// bf16 stored as its raw 16 bits.
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}
// Round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Element loads/stores by storage type: float, or uint16_t holding bf16.
__device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld(const uint16_t* p, int64_t i) { return bf16_bits_to_f32(p[i]); }
__device__ __forceinline__ void st(float* p, int64_t i, float x) { p[i] = x; }
__device__ __forceinline__ void st(uint16_t* p, int64_t i, float x) { p[i] = f32_to_bf16_bits(x); }

// v_mfma_f32_16x16x32_{f16,bf16}: D(16x16) += A(16x32) B(32x16).
//   A: lane l holds row (l & 15), eight K slots of K-group (l >> 4).
//   B: lane l holds column (l & 15), the same eight K slots of K-group (l >> 4).
//   D: lane l holds rows 4*(l >> 4) + i (i = 0..3) of column (l & 15).
// Which of the 32 K indices sits in which (group, slot) only has to agree between A and
// B. Every operand in libkda uses the map below, which makes two D tiles stacked along K
// (rows 0-15 and 16-31 of a 32-row block) directly usable as a B operand: slot i < 4 is
// row 4g+i of the first tile, slot i >= 4 is row 4g+i-4 of the second.
__device__ __forceinline__ int kslot(int g, int i) { return (i < 4) ? (4 * g + i) : (12 + 4 * g + i); }

__device__ __forceinline__ floatx4 mfma_f16(const half8& a, const half8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma_bf16(const bf16x8& a, const bf16x8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Split x into a bf16 pair with hi + lo = x to about 16 significant bits.
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
  hi = static_cast<__bf16>(x);
  lo = static_cast<__bf16>(x - static_cast<float>(hi));
}
// Split x into an fp16 pair with hi + lo = x to about 22 significant bits.
__device__ __forceinline__ void split_f16(float x, _Float16& hi, _Float16& lo) {
  hi = static_cast<_Float16>(x);
  lo = static_cast<_Float16>(x - static_cast<float>(hi));
}

}  // namespace kda
