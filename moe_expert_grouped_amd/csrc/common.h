// common.h -- device helpers shared by the HIP kernels of the MoE library
// (gfx950 / CDNA4 only).  Nothing here is shared with the oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_LDS __attribute__((address_space(3)))

namespace moe {

constexpr int kWave = 64;      // CDNA wavefront width
constexpr int kRowBlock = 128; // rows per task / expert alignment unit

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// fp32 -> bf16 with round-to-nearest-even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> IEEE half, round-to-nearest-even (the hardware conversion).
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
  _Float16 h = (_Float16)f;
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

} // namespace moe
