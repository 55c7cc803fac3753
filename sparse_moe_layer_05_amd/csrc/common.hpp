// Device-side helpers shared by the gfx950 kernels of the MoE layer library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4_t;

constexpr int kWave = 64;
constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, 32 CUs each, one L2 per die

// bf16 <-> fp32. bf16 is the upper half of a binary32; the narrowing rounds to nearest even
// (inputs are finite).
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t u16) {
  return __uint_as_float(u16 << 16);
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
// Two fp32 -> packed bf16x2 (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Two fp32 -> two OCP e4m3 codes (round to nearest even) in the low 16 bits.
__device__ __forceinline__ uint32_t cvt_fp8x2(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

__device__ __forceinline__ float sqrelu(float a) { return a > 0.f ? a * a : 0.f; }

__host__ __device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

// Hardware hands workgroup b to die b % 8. Remap so each die walks one contiguous range of
// logical tiles: neighbouring tiles (which share weight or activation panels) then share an L2.
// nblk must be a multiple of 8.
__device__ __forceinline__ int xcd_logical_block(int b, int nblk) {
  return (b % kXcds) * (nblk / kXcds) + b / kXcds;
}

}  // namespace moe
