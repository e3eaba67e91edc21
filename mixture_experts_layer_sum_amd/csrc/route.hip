// Router: logits = hidden . W_router (+ bias), top-k per token, softmax over
// the k selected logits, and the per-expert token histogram.
//
// cf-1.com/news/5914943 §2.1: the router is one small linear layer; the k
// best-scoring experts are kept and their scores softmax-normalised.
// 2kiu.com/news/2885792 §3.1: logits = einsum('bsd,de->bse', hidden, router_w).
// 2kiu.com/news/2885792 §5.3: equal logits are ranked by ascending expert id.
// cf-1.com/news/5914943 §2.3: tokens_per_expert counts the router's choices.
//
// One block = 64 tokens, 4 waves; wave w owns tokens 16w..16w+15 of the block.
// bf16: the logits tile is a chain of 16x16x32 MFMAs whose A operand (hidden
// rows) streams from HBM straight into registers (each hidden element is used
// by exactly one wave) and whose B operand (W_router, k-contiguous after an
// in-register 4x8 transpose) is staged per k-chunk in LDS and shared by the
// four waves.  The epilogue keeps the tile in LDS, and each wave runs k rounds
// of a wave64 argmax reduction per token.
#include "common.hpp"
#include "internal.hpp"

namespace moe {

constexpr int kRtTok = 64;
constexpr int kRtThreads = 256;

__global__ void zero_i32_kernel(int32_t* __restrict__ p, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// Top-k + softmax + histogram for the rows of one wave.  lg: LDS tile
// [64][ldl] of fp32 logits (bias included).  Ordering: larger logit first,
// lower expert id first among equal logits.
__device__ __forceinline__ void topk_rows(const float* lg, int ldl, int t0, int T, int N, int k,
                                          int32_t* __restrict__ topk_idx,
                                          float* __restrict__ topk_w, int* hist) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int rr = 0; rr < 16; ++rr) {
    const int r = w * 16 + rr;
    const int t = t0 + r;
    if (t >= T) break;
    float v[4];
    unsigned taken = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = lane + 64 * c;
      v[c] = (e < N) ? lg[r * ldl + e] : 0.f;
      if (e >= N) taken |= 1u << c;
    }
    float sv[4] = {0.f, 0.f, 0.f, 0.f};
    int si[4] = {0, 0, 0, 0};
    float vmax = 0.f;
    for (int j = 0; j < k; ++j) {
      float bv = -INFINITY;
      int be = 0x7fffffff;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (!(taken & (1u << c))) {
          const int e = lane + 64 * c;
          if (be == 0x7fffffff || v[c] > bv) { bv = v[c]; be = e; }
        }
      }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        const float ov = __shfl_xor(bv, m, 64);
        const int oe = __shfl_xor(be, m, 64);
        if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
      }
      if ((be & 63) == lane) taken |= 1u << (be >> 6);
      if (j == 0) vmax = bv;
      if ((j & 63) == lane) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (c == (j >> 6)) { sv[c] = bv; si[c] = be; }
      }
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (lane + 64 * c < k) s += __expf(sv[c] - vmax);
    s = wave_sum(s);
    const float inv = 1.f / s;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = lane + 64 * c;
      if (j < k) {
        topk_idx[(size_t)t * k + j] = si[c];
        topk_w[(size_t)t * k + j] = __expf(sv[c] - vmax) * inv;
        atomicAdd(&hist[si[c]], 1);
      }
    }
  }
}

template <int NT>
struct RouterCfg {
  static constexpr int Npad = 16 * NT;
  static constexpr int BK = NT <= 4 ? 256 : (NT == 8 ? 128 : 64);
  static constexpr int ldw = BK + 8;                     // bf16 elements per LDS row of W^T
  static constexpr int ldl = Npad + 1;                   // floats per LDS row of logits
  static constexpr int w_bytes = Npad * ldw * 2;
  static constexpr int l_bytes = kRtTok * ldl * 4;
  static constexpr int smem = w_bytes > l_bytes ? w_bytes : l_bytes;
};

template <int NT>
__global__ __launch_bounds__(kRtThreads) void router_bf16_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, int T, int d, int N, int k, float* __restrict__ logits,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int32_t* __restrict__ counts) {
  using C = RouterCfg<NT>;
  constexpr int BK = C::BK, ldw = C::ldw, NS = BK / 32;
  __shared__ __align__(16) unsigned char smem[C::smem];
  __shared__ int hist[256];
  uint16_t* Ws = reinterpret_cast<uint16_t*>(smem);
  float* lg = reinterpret_cast<float*>(smem);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int t0 = blockIdx.x * kRtTok;
  const int g = lane >> 4, ml = lane & 15;
  const int row = t0 + w * 16 + ml;
  const bool rv = row < T;
  const uint16_t* hrow = hidden + (size_t)(rv ? row : 0) * d + 8 * g;
  for (int i = tid; i < 256; i += kRtThreads) hist[i] = 0;

  f32x4 acc[NT];
#pragma unroll
  for (int c = 0; c < NT; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint4 z4 = make_uint4(0, 0, 0, 0);
  uint4 a[NS];
  {
    const int klen = d < BK ? d : BK;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      a[s] = (rv && 32 * s < klen) ? *reinterpret_cast<const uint4*>(hrow + 32 * s) : z4;
  }
  const bool nvec = (N & 7) == 0;
  for (int k0 = 0; k0 < d; k0 += BK) {
    const int klen = (d - k0) < BK ? (d - k0) : BK;
    __syncthreads();
    // Stage W_router rows [k0, k0+klen) transposed: Ws[n][kk] (k contiguous).
    const int kq_n = klen >> 2, cg_n = C::Npad >> 3;
    for (int it = tid; it < kq_n * cg_n; it += kRtThreads) {
      const int kq = it % kq_n, cg = it / kq_n;
      uint32_t r[4][4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int kk = k0 + 4 * kq + q;
        const uint16_t* src = wr + (size_t)kk * N + 8 * cg;
        if (nvec) {
          uint4 x = (8 * cg < N) ? *reinterpret_cast<const uint4*>(src) : z4;
          r[q][0] = x.x; r[q][1] = x.y; r[q][2] = x.z; r[q][3] = x.w;
        } else {
          uint16_t e8[8];
#pragma unroll
          for (int c = 0; c < 8; ++c) e8[c] = (8 * cg + c < N) ? src[c] : (uint16_t)0;
#pragma unroll
          for (int c = 0; c < 4; ++c) r[q][c] = e8[2 * c] | ((uint32_t)e8[2 * c + 1] << 16);
        }
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int h = c >> 1;
        uint32_t lo, hi;
        if (c & 1) {
          lo = (r[0][h] >> 16) | (r[1][h] & 0xFFFF0000u);
          hi = (r[2][h] >> 16) | (r[3][h] & 0xFFFF0000u);
        } else {
          lo = (r[0][h] & 0xFFFFu) | (r[1][h] << 16);
          hi = (r[2][h] & 0xFFFFu) | (r[3][h] << 16);
        }
        *reinterpret_cast<uint2*>(Ws + (8 * cg + c) * ldw + 4 * kq) = make_uint2(lo, hi);
      }
    }
    __syncthreads();
    uint4 an[NS];
    const int kn = k0 + BK;
    const int klen_n = (d - kn) < BK ? (d - kn) : BK;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      an[s] = (rv && kn < d && 32 * s < klen_n) ? *reinterpret_cast<const uint4*>(hrow + kn + 32 * s) : z4;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (32 * s < klen) {
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          const uint4 b = *reinterpret_cast<const uint4*>(Ws + (16 * c + ml) * ldw + 32 * s + 8 * g);
          acc[c] = mfma16(a[s], b, acc[c]);
        }
      }
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) a[s] = an[s];
  }
  __syncthreads();   // every wave is done with Ws; reuse the space for the logits tile
#pragma unroll
  for (int c = 0; c < NT; ++c) {
    const int col = 16 * c + ml;
    const float b = (bias != nullptr && col < N) ? bias[col] : 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) lg[(w * 16 + 4 * g + r) * C::ldl + col] = acc[c][r] + b;
  }
  __syncthreads();
  for (int i = tid; i < kRtTok * N; i += kRtThreads) {
    const int r = i / N, e = i - r * N;
    if (t0 + r < T) logits[(size_t)(t0 + r) * N + e] = lg[r * C::ldl + e];
  }
  topk_rows(lg, C::ldl, t0, T, N, k, topk_idx, topk_w, hist);
  __syncthreads();
  for (int e = tid; e < N; e += kRtThreads)
    if (hist[e]) atomicAdd(&counts[e], hist[e]);
}

// fp32: the same epilogue after a plain fp32 dot product per (token, expert).
__global__ __launch_bounds__(kRtThreads) void router_f32_kernel(
    const float* __restrict__ hidden, const float* __restrict__ wr, const float* __restrict__ bias,
    int T, int d, int N, int k, float* __restrict__ logits, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, int32_t* __restrict__ counts) {
  __shared__ float lg[kRtTok * 257];
  __shared__ int hist[256];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kRtTok;
  const int ldl = N + 1;
  for (int i = tid; i < 256; i += kRtThreads) hist[i] = 0;
  for (int i = tid; i < kRtTok * N; i += kRtThreads) {
    const int r = i / N, e = i - r * N;
    const int t = t0 + r;
    float s = 0.f;
    if (t < T) {
      const float* h = hidden + (size_t)t * d;
      for (int q = 0; q < d; ++q) s = fmaf(h[q], wr[(size_t)q * N + e], s);
      s += bias ? bias[e] : 0.f;
      logits[(size_t)t * N + e] = s;
    }
    lg[r * ldl + e] = s;
  }
  __syncthreads();
  topk_rows(lg, ldl, t0, T, N, k, topk_idx, topk_w, hist);
  __syncthreads();
  for (int e = tid; e < N; e += kRtThreads)
    if (hist[e]) atomicAdd(&counts[e], hist[e]);
}

hipError_t launch_route(const void* hidden, const void* w_router, const float* bias, int T, int d,
                        int N, int k, bool bf16, float* logits, int32_t* topk_idx, float* topk_w,
                        int32_t* counts, hipStream_t stream) {
  hipLaunchKernelGGL(zero_i32_kernel, dim3((N + 255) / 256), dim3(256), 0, stream, counts, N);
  const dim3 grid((T + kRtTok - 1) / kRtTok), block(kRtThreads);
  if (!bf16) {
    hipLaunchKernelGGL(router_f32_kernel, grid, block, 0, stream,
                       static_cast<const float*>(hidden), static_cast<const float*>(w_router),
                       bias, T, d, N, k, logits, topk_idx, topk_w, counts);
    return hipGetLastError();
  }
  const auto* h = static_cast<const uint16_t*>(hidden);
  const auto* wr = static_cast<const uint16_t*>(w_router);
  const int nt = (N + 15) / 16;
#define MOE_ROUTER_CASE(NTV)                                                                   \
  hipLaunchKernelGGL(router_bf16_kernel<NTV>, grid, block, 0, stream, h, wr, bias, T, d, N, k, \
                     logits, topk_idx, topk_w, counts)
  if (nt <= 1) MOE_ROUTER_CASE(1);
  else if (nt <= 2) MOE_ROUTER_CASE(2);
  else if (nt <= 4) MOE_ROUTER_CASE(4);
  else if (nt <= 8) MOE_ROUTER_CASE(8);
  else MOE_ROUTER_CASE(16);
#undef MOE_ROUTER_CASE
  return hipGetLastError();
}

}  // namespace moe
