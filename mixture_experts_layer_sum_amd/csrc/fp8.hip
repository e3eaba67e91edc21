// FP8 (OCP E4M3) expert weights for decode-shaped batches.
//
// cf-1.com/news/5914943 §3.1: MoE experts are stored in FP8 to cut the memory
// their weights take.  At decode the layer's time is reading the active
// experts' weights (hotelren.com/news/3071227 §2.2 and §2.3: only the
// selected experts' weights are touched), so one byte per weight instead of
// two halves the traffic.
//
// Format: OCP FP8 E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa
// bits, subnormals, largest finite 448, no infinity).  Per output column of
// each expert matrix: scale = amax / 448 (1 for an all-zero column) and
// code = RNE(w / scale) clamped to +-448, both divisions IEEE float32.  The
// gfx950 conversion v_cvt_pk_fp8_f32 rounds to nearest even but turns values
// past the finite range into NaN, hence the clamp.
//
// Layer: the weight-streaming kernel of the bf16 path (32-row tiles, 32x32x16
// bf16 MFMAs, column-permuted B operands) reading 8 bytes (8 columns) per lane
// per weight row instead of 16: the codes are widened to bf16 exactly
// (v_cvt_scalef32_pk_bf16_fp8 with scale 1; every E4M3 value is a bf16
// value), multiplied in the MFMA, and the column scale is applied to the fp32
// sums in the epilogue (before the SwiGLU for the up projection).
#include "common.hpp"
#include "internal.hpp"

namespace moe {

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- quantisation
// Block (expert e, 256 consecutive columns); thread = column; two passes over K.
template <bool BF16>
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const void* __restrict__ w, int K, int M,
                                                           uint8_t* __restrict__ q,
                                                           float* __restrict__ scale) {
  const int e = blockIdx.y;
  const int m = blockIdx.x * 256 + threadIdx.x;
  if (m >= M) return;
  const size_t base = (size_t)e * K * M + m;
  auto value = [&](int k) -> float {
    if (BF16) return bf16_to_f32(static_cast<const uint16_t*>(w)[base + (size_t)k * M]);
    return static_cast<const float*>(w)[base + (size_t)k * M];
  };
  float amax = 0.f;
  for (int k = 0; k < K; ++k) amax = fmaxf(amax, fabsf(value(k)));
  const float s = amax > 0.f ? __fdiv_rn(amax, 448.f) : 1.f;
  scale[(size_t)e * M + m] = s;
  for (int k = 0; k < K; ++k) {
    float r = __fdiv_rn(value(k), s);
    r = fminf(fmaxf(r, -448.f), 448.f);
    const int packed = __builtin_amdgcn_cvt_pk_fp8_f32(r, 0.f, 0, false);
    q[base + (size_t)k * M] = static_cast<uint8_t>(packed & 0xFF);
  }
}

hipError_t launch_quantize_fp8(const void* w, bool bf16, int N, int K, int M, uint8_t* q,
                               float* scale, hipStream_t stream) {
  const dim3 grid((M + 255) / 256, N);
  if (bf16)
    hipLaunchKernelGGL(quantize_fp8_kernel<true>, grid, dim3(256), 0, stream, w, K, M, q, scale);
  else
    hipLaunchKernelGGL(quantize_fp8_kernel<false>, grid, dim3(256), 0, stream, w, K, M, q, scale);
  return hipGetLastError();
}

// ---------------------------------------------------------------- weight streaming
// 8 codes (one 8-byte load) -> 8 bf16 (one MFMA-sized 16-byte vector), exact.
__device__ __forceinline__ uint4 widen8(uint2 c) {
  const bf16x2v a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c.x, 1.0f, false);
  const bf16x2v b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c.x, 1.0f, true);
  const bf16x2v d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c.y, 1.0f, false);
  const bf16x2v f = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c.y, 1.0f, true);
  return make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                    __builtin_bit_cast(uint32_t, d), __builtin_bit_cast(uint32_t, f));
}

typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 load_stream8(const uint8_t* p) {
  const u32x2v v = __builtin_nontemporal_load(reinterpret_cast<const u32x2v*>(p));
  return make_uint2(v.x, v.y);
}

// A wave owns (expert, 32 rows, column slice).  Lane 32h + i loads k-rows
// k0 + 8h .. +7 of its 8 columns; UP: lanes i < 16 read W1 columns n0 + 8i,
// lanes i >= 16 the same columns of W3 (128 activation columns per wave);
// DOWN: lane i reads W2 columns n0 + 8i (256 columns).
template <bool UP>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 8)))
void grouped_gemm_fp8_rows32_kernel(const uint16_t* __restrict__ X,
                                    const int32_t* __restrict__ offsets, int N,
                                    const uint8_t* __restrict__ Qa, const uint8_t* __restrict__ Qb,
                                    const float* __restrict__ Sa, const float* __restrict__ Sb,
                                    int K, int Nout, int n_slices, int max_rows,
                                    void* __restrict__ out) {
  const int mt = blockIdx.x / n_slices, ns = blockIdx.x - mt * n_slices;
  int e, r0, rend;
  if (!find_tile(offsets, N, mt, 32, max_rows, e, r0, rend)) return;
  e = __builtin_amdgcn_readfirstlane(e);
  r0 = __builtin_amdgcn_readfirstlane(r0);
  rend = __builtin_amdgcn_readfirstlane(rend);

  const int lane = threadIdx.x, i = lane & 31, h = lane >> 5;
  const int n0 = ns * (UP ? 128 : 256);
  const int col = UP ? n0 + 8 * (i & 15) : n0 + 8 * i;
  const size_t wexp = (size_t)e * K * Nout;
  const uint8_t* wsrc = (UP && i >= 16 ? Qb : Qa) + wexp + col + (size_t)(8 * h) * Nout;
  const float* srow = (UP && i >= 16 ? Sb : Sa) + (size_t)e * Nout + col;
  const uint16_t* asrc = X + (size_t)min(r0 + i, rend - 1) * K + 8 * h;

  f32x16 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;

  const size_t rstride = (size_t)Nout;
  uint2 wb[2][8];
  uint4 xa[2];
#define MOE_F8_LOAD(S, k0)                                                            \
  do {                                                                               \
    _Pragma("unroll") for (int kk = 0; kk < 8; ++kk)                                 \
        wb[S][kk] = load_stream8(wsrc + (size_t)((k0) + kk) * rstride);              \
    xa[S] = *reinterpret_cast<const uint4*>(asrc + (k0));                            \
  } while (0)
#define MOE_F8_MMA(S)                                                                 \
  do {                                                                               \
    uint4 rows_[8], bf[8];                                                           \
    _Pragma("unroll") for (int kk = 0; kk < 8; ++kk) rows_[kk] = widen8(wb[S][kk]);  \
    transpose8x8(rows_, bf);                                                         \
    _Pragma("unroll") for (int c = 0; c < 8; ++c) acc[c] = mfma32(xa[S], bf[c], acc[c]); \
  } while (0)

  const int nk = K / 16;                        // K is a multiple of 64: nk is even
  MOE_F8_LOAD(0, 0);
  for (int kt = 0; kt < nk; kt += 2) {
    MOE_F8_LOAD(1, (kt + 1) * 16);
    MOE_F8_MMA(0);
    if (kt + 2 < nk) MOE_F8_LOAD(0, (kt + 2) * 16);
    MOE_F8_MMA(1);
  }
#undef MOE_F8_LOAD
#undef MOE_F8_MMA

  float sc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) sc[c] = srow[c];

  // acc[c][r]: row r0 + 8 (r / 4) + 4h + r % 4, column col + c
  if (UP) {
    uint16_t* act = static_cast<uint16_t*>(out);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float v[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float mine = acc[c][r] * sc[c];
        const float other = __shfl_xor(mine, 16, 64);    // W3 half for lanes i < 16
        v[c] = mine * __builtin_amdgcn_rcpf(1.f + __expf(-mine)) * other;
      }
      const int row = r0 + 8 * (r >> 2) + 4 * h + (r & 3);
      if (i < 16 && row < rend) {
        const uint4 pk = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                    pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
        *reinterpret_cast<uint4*>(act + (size_t)row * Nout + col) = pk;
      }
    }
  } else {
    float* y = static_cast<float*>(out);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = r0 + 8 * (r >> 2) + 4 * h + (r & 3);
      if (row < rend) {
        float4* dst = reinterpret_cast<float4*>(y + (size_t)row * Nout + col);
        dst[0] = make_float4(acc[0][r] * sc[0], acc[1][r] * sc[1], acc[2][r] * sc[2],
                             acc[3][r] * sc[3]);
        dst[1] = make_float4(acc[4][r] * sc[4], acc[5][r] * sc[5], acc[6][r] * sc[6],
                             acc[7][r] * sc[7]);
      }
    }
  }
}

// Up projection in wave pairs: a block of two waves owns (expert, 32 rows, 256
// activation columns); wave 0 streams those columns' W1 codes and wave 1 their
// W3 codes (32 lanes x 8 bytes = 256 contiguous bytes of a k-row, twice the
// piece of the one-wave layout above), and the scaled SwiGLU halves meet in
// LDS: wave 0 hands over its W1 sums of the upper 16 accumulator rows, wave 1
// its W3 sums of the lower 16, and each wave finishes and stores half.
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2, 8)))
void grouped_gemm_fp8_rows32_up2_kernel(const uint16_t* __restrict__ X,
                                        const int32_t* __restrict__ offsets, int N,
                                        const uint8_t* __restrict__ Q1, const uint8_t* __restrict__ Q3,
                                        const float* __restrict__ S1, const float* __restrict__ S3,
                                        int K, int F, int n_slices, int max_rows,
                                        uint16_t* __restrict__ act) {
  __shared__ float xch[2][8 * 8 * 64];      // [wave that wrote][c][half-row r][lane]
  const int mt = blockIdx.x / n_slices, ns = blockIdx.x - mt * n_slices;
  int e, r0, rend;
  if (!find_tile(offsets, N, mt, 32, max_rows, e, r0, rend)) return;
  e = __builtin_amdgcn_readfirstlane(e);
  r0 = __builtin_amdgcn_readfirstlane(r0);
  rend = __builtin_amdgcn_readfirstlane(rend);

  const int lane = threadIdx.x & 63, i = lane & 31, h = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int col = ns * 256 + 8 * i;
  const uint8_t* wsrc = (w == 0 ? Q1 : Q3) + (size_t)e * K * F + col + (size_t)(8 * h) * F;
  const float* srow = (w == 0 ? S1 : S3) + (size_t)e * F + col;
  const uint16_t* asrc = X + (size_t)min(r0 + i, rend - 1) * K + 8 * h;

  f32x16 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;

  const size_t rstride = (size_t)F;
  uint2 wb[2][8];
  uint4 xa[2];
#define MOE_F8U_LOAD(S, k0)                                                           \
  do {                                                                               \
    _Pragma("unroll") for (int kk = 0; kk < 8; ++kk)                                 \
        wb[S][kk] = load_stream8(wsrc + (size_t)((k0) + kk) * rstride);              \
    xa[S] = *reinterpret_cast<const uint4*>(asrc + (k0));                            \
  } while (0)
#define MOE_F8U_MMA(S)                                                                \
  do {                                                                               \
    uint4 rows_[8], bf[8];                                                           \
    _Pragma("unroll") for (int kk = 0; kk < 8; ++kk) rows_[kk] = widen8(wb[S][kk]);  \
    transpose8x8(rows_, bf);                                                         \
    _Pragma("unroll") for (int c = 0; c < 8; ++c) acc[c] = mfma32(xa[S], bf[c], acc[c]); \
  } while (0)

  const int nk = K / 16;                        // K is a multiple of 64: nk is even
  MOE_F8U_LOAD(0, 0);
  for (int kt = 0; kt < nk; kt += 2) {
    MOE_F8U_LOAD(1, (kt + 1) * 16);
    MOE_F8U_MMA(0);
    if (kt + 2 < nk) MOE_F8U_LOAD(0, (kt + 2) * 16);
    MOE_F8U_MMA(1);
  }
#undef MOE_F8U_LOAD
#undef MOE_F8U_MMA

  float sc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) sc[c] = srow[c];

  // acc[c][r]: row r0 + 8 (r / 4) + 4h + r % 4, column col + c.  Wave 0 keeps
  // r < 8 and hands over r >= 8; wave 1 the other way round.
  const int keep = (w == 0) ? 0 : 8;
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const float v = ((w == 0) ? acc[c][8 + rr] : acc[c][rr]) * sc[c];
      xch[w][(c * 8 + rr) * 64 + lane] = v;
    }
  __syncthreads();
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) {
    float v[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float mine = ((w == 0) ? acc[c][rr] : acc[c][8 + rr]) * sc[c];
      const float other = xch[1 - w][(c * 8 + rr) * 64 + lane];
      const float g1 = (w == 0) ? mine : other, g3 = (w == 0) ? other : mine;
      v[c] = g1 * __builtin_amdgcn_rcpf(1.f + __expf(-g1)) * g3;
    }
    const int r = keep + rr;
    const int row = r0 + 8 * (r >> 2) + 4 * h + (r & 3);
    if (row < rend) {
      const uint4 pk = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                  pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
      *reinterpret_cast<uint4*>(act + (size_t)row * F + col) = pk;
    }
  }
}

bool fp8_rows_supported(int max_rows, int N) { return (max_rows + N - 1) / N <= 32; }

hipError_t launch_expert_up_fp8(const void* x_perm, const int32_t* offsets, const uint8_t* w1q,
                                const uint8_t* w3q, const float* s1, const float* s3, int N,
                                int d, int f, int max_rows, void* act, hipStream_t stream) {
  const int m_bound = (max_rows + 31) / 32 + N;
  if (f % 256 == 0) {
    const int n_slices = f / 256;
    hipLaunchKernelGGL(grouped_gemm_fp8_rows32_up2_kernel, dim3(m_bound * n_slices), dim3(128), 0,
                       stream, static_cast<const uint16_t*>(x_perm), offsets, N, w1q, w3q, s1, s3,
                       d, f, n_slices, max_rows, static_cast<uint16_t*>(act));
    return hipGetLastError();
  }
  const int n_slices = f / 128;
  hipLaunchKernelGGL(grouped_gemm_fp8_rows32_kernel<true>, dim3(m_bound * n_slices), dim3(64), 0,
                     stream, static_cast<const uint16_t*>(x_perm), offsets, N, w1q, w3q, s1, s3, d,
                     f, n_slices, max_rows, act);
  return hipGetLastError();
}

hipError_t launch_expert_down_fp8(const void* act, const int32_t* offsets, const uint8_t* w2q,
                                  const float* s2, int N, int d, int f, int max_rows,
                                  float* y_perm, hipStream_t stream) {
  const int n_slices = d / 256;
  const int m_bound = (max_rows + 31) / 32 + N;
  hipLaunchKernelGGL(grouped_gemm_fp8_rows32_kernel<false>, dim3(m_bound * n_slices), dim3(64), 0,
                     stream, static_cast<const uint16_t*>(act), offsets, N, w2q,
                     static_cast<const uint8_t*>(nullptr), s2, static_cast<const float*>(nullptr), f,
                     d, n_slices, max_rows, static_cast<void*>(y_perm));
  return hipGetLastError();
}

}  // namespace moe
