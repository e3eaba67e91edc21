// Shared device helpers for the gfx950 MoE kernels: bf16 conversion, MFMA
// operand types and wave64 reductions.  Nothing here is shared with the CPU
// oracle.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// bf16 bit pattern -> float (exact widening).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float -> bf16 bit pattern, round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// One 16x16x32 bf16 MFMA step: acc += A(16x32) * B(32x16).
// Operand convention used by every kernel here: lane l holds row/column
// (l % 16) and the 8 consecutive k values 8*(l/16) .. 8*(l/16)+7.  The result
// lane l, element r is D[4*(l/16) + r][l % 16].
__device__ __forceinline__ f32x4 mfma16(const uint4& a, const uint4& b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

template <typename T>
__device__ __forceinline__ T wave_shfl_xor(T v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

}  // namespace moe
