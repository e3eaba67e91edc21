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

// One 32x32x16 bf16 MFMA step: lane l holds row/column (l % 32) and k values
// 8*(l/32) .. +7; result lane l, element r is D[8*(r/4) + 4*(l/32) + r%4][l % 32].
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(const uint4& a, const uint4& b, f32x16 acc) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
// Streaming 16-byte load (weights are read once): non-temporal hint.
__device__ __forceinline__ uint4 load_stream(const uint16_t* p) {
  const u32x4v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void transpose8x8(const uint4 (&r)[8], uint4 (&c)[8]) {
  // r[kk] holds columns 0..7 of k-row kk; c[col] gets k-rows 0..7 of column col
  uint32_t w[8][4];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    w[kk][0] = r[kk].x; w[kk][1] = r[kk].y; w[kk][2] = r[kk].z; w[kk][3] = r[kk].w;
  }
#pragma unroll
  for (int col = 0; col < 8; ++col) {
    const int h = col >> 1;
    uint32_t o[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t lo = w[2 * m][h], hi = w[2 * m + 1][h];
      o[m] = (col & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
    }
    c[col] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// Row tiles of `bm` rows are numbered expert by expert.  Offsets are clamped
// to [0, max_rows] and made non-decreasing, so inconsistent offsets can never
// address a row >= max_rows.  Wave-uniform.
__device__ __forceinline__ int count_tiles(const int32_t* __restrict__ offsets, int N, int bm,
                                           int max_rows) {
  const int lane = threadIdx.x & 63;
  int total = 0;
  for (int b = 0; b < N; b += 64) {
    const int e = b + lane;
    int cnt = 0;
    if (e < N) {
      const int o0 = min(max(offsets[e], 0), max_rows);
      const int o1 = min(max(offsets[e + 1], o0), max_rows);
      cnt = (o1 - o0 + bm - 1) / bm;
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) cnt += __shfl_xor(cnt, m, 64);
    total += cnt;
  }
  return total;
}

// Locate row tile `mt`; returns false if mt is past the last tile.
__device__ __forceinline__ bool find_tile(const int32_t* __restrict__ offsets, int N, int mt,
                                          int bm, int max_rows, int& e_out, int& r0, int& rend) {
  const int lane = threadIdx.x & 63;
  int before = 0;
  for (int b = 0; b < N; b += 64) {
    const int e = b + lane;
    int o0 = 0, o1 = 0;
    if (e < N) {
      o0 = min(max(offsets[e], 0), max_rows);
      o1 = min(max(offsets[e + 1], o0), max_rows);
    }
    const int cnt = (o1 - o0 + bm - 1) / bm;
    int inc = cnt;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const int v = __shfl_up(inc, m, 64);
      if (lane >= m) inc += v;
    }
    const int total = __shfl(inc, 63, 64);
    if (mt < before + total) {
      const unsigned long long bal = __ballot(before + inc > mt);
      const int L = __ffsll(static_cast<long long>(bal)) - 1;
      const int exc = __shfl(inc - cnt, L, 64);
      e_out = b + L;
      r0 = __shfl(o0, L, 64) + (mt - before - exc) * bm;
      rend = __shfl(o1, L, 64);
      return true;
    }
    before += total;
  }
  return false;
}


}  // namespace moe
