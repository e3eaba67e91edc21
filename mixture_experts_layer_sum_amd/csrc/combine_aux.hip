// Weighted combine back to token order, and the load-balancing loss.
//
// Combine -- cf-1.com/news/5914943 §2.1: the layer output is the gate-weighted
// sum of the selected experts' outputs; devpress.csdn.net/awstech/6a91abf4...
// §4.1: gather the expert results back to token order.  Summed in slot order
// in fp32; dropped slots add nothing and nothing is renormalised.
// hotelren.com/news/5904824 §3.3: shared experts, called by every token, are
// added with weight 1.
//
// Aux loss -- cf-1.com/news/5914943 §2.3 and hotelren.com/news/5904824 §3.2:
// aux = N * sum_e f_e * P_e with f_e the share of router assignments at e
// (pre-drop counts / (T*k)) and P_e the mean full-N softmax probability.
// All reductions run in a fixed order (no float atomics), so the result is
// bitwise reproducible.
#include "common.hpp"
#include "internal.hpp"

namespace moe {

// One block per token; each thread owns 4 consecutive columns.  The shared
// experts' outputs (y_shared [n_shared][T][d]) are added after the routed
// slots, in shared-expert order.
template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_perm,
                                                      const int32_t* __restrict__ slot_row,
                                                      const float* __restrict__ topk_w,
                                                      const float* __restrict__ y_shared,
                                                      int n_shared, int T, int d, int k,
                                                      void* __restrict__ y) {
  __shared__ int srow[256];
  __shared__ float sw[256];
  const int t = blockIdx.x;
  for (int j = threadIdx.x; j < k; j += blockDim.x) {
    srow[j] = slot_row[(size_t)t * k + j];
    sw[j] = topk_w[(size_t)t * k + j];
  }
  __syncthreads();
  // four column groups per pass, so that each slot's four loads are in flight together
  const int nv = d >> 2;
  for (int v0 = threadIdx.x; v0 < nv; v0 += 4 * blockDim.x) {
    float4 acc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
      const int r = srow[j];
      if (r < 0) continue;
      const float wj = sw[j];
      const float4* src = reinterpret_cast<const float4*>(y_perm + (size_t)r * d);
      float4 x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int v = v0 + u * blockDim.x;
        x[u] = v < nv ? src[v] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        acc[u].x = fmaf(wj, x[u].x, acc[u].x);
        acc[u].y = fmaf(wj, x[u].y, acc[u].y);
        acc[u].z = fmaf(wj, x[u].z, acc[u].z);
        acc[u].w = fmaf(wj, x[u].w, acc[u].w);
      }
    }
    for (int q = 0; q < n_shared; ++q) {
      const float4* src = reinterpret_cast<const float4*>(y_shared + ((size_t)q * T + t) * d);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int v = v0 + u * blockDim.x;
        if (v < nv) {
          const float4 x = src[v];
          acc[u].x += x.x;
          acc[u].y += x.y;
          acc[u].z += x.z;
          acc[u].w += x.w;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int v = v0 + u * blockDim.x;
      if (v >= nv) continue;
      if (BF16) {
        reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + (size_t)t * d)[v] =
            make_uint2(pack_bf16x2(acc[u].x, acc[u].y), pack_bf16x2(acc[u].z, acc[u].w));
      } else {
        reinterpret_cast<float4*>(static_cast<float*>(y) + (size_t)t * d)[v] = acc[u];
      }
    }
  }
}

hipError_t launch_combine(const float* y_perm, const int32_t* slot_row, const float* topk_w,
                          const float* y_shared, int n_shared, int T, int d, int k, bool bf16,
                          void* y, hipStream_t stream) {
  if (bf16)
    hipLaunchKernelGGL(combine_kernel<true>, dim3(T), dim3(256), 0, stream, y_perm, slot_row,
                       topk_w, y_shared, n_shared, T, d, k, y);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3(T), dim3(256), 0, stream, y_perm, slot_row,
                       topk_w, y_shared, n_shared, T, d, k, y);
  return hipGetLastError();
}

constexpr int kAuxTok = 16;    // tokens per block (4 per wave)

// part[b][e] = sum over the block's tokens of softmax(logits[t])_e, in token
// order.  A wave loads its 4 tokens' logits before reducing any of them.
__global__ __launch_bounds__(256) void aux_partial_kernel(const float* __restrict__ logits, int T,
                                                          int N, float* __restrict__ part) {
  constexpr int TPW = kAuxTok / 4;
  __shared__ float red[4][256];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int tb = blockIdx.x * kAuxTok + w * TPW;
  float v[TPW][4];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int t = tb + i;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = lane + 64 * c;
      v[i][c] = (t < T && e < N) ? logits[(size_t)t * N + e] : -INFINITY;
    }
  }
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    if (tb + i >= T) break;
    float m = fmaxf(fmaxf(v[i][0], v[i][1]), fmaxf(v[i][2], v[i][3]));
    m = wave_max(m);
    float s = 0.f;
    float p[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      p[c] = (lane + 64 * c < N) ? __expf(v[i][c] - m) : 0.f;
      s += p[c];
    }
    s = wave_sum(s);
    const float inv = 1.f / s;
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] += p[c] * inv;
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) red[w][lane + 64 * c] = acc[c];
  __syncthreads();
  for (int e = threadIdx.x; e < N; e += 256)
    part[(size_t)blockIdx.x * N + e] = ((red[0][e] + red[1][e]) + red[2][e]) + red[3][e];
}

// Single block: P_e = sum_b part[b][e] / T, then aux = N * sum_e f_e P_e.
// The 1024 threads split the blocks: expert e is summed by G = 1024 / N' threads
// (N' = N rounded up to a power of two), thread g taking blocks g, g + G, ...;
// the G partial sums then meet in a fixed tree, so the order never changes.
constexpr int kAuxFinal = 1024;
__global__ __launch_bounds__(kAuxFinal) void aux_final_kernel(const float* __restrict__ part, int nb,
                                                        const int32_t* __restrict__ counts, int T,
                                                        int N, int k, float* __restrict__ aux) {
  __shared__ double red[kAuxFinal];
  __shared__ float term[256];
  const int tid = threadIdx.x;
  int np2 = 1;
  while (np2 < N) np2 <<= 1;
  const int G = kAuxFinal / np2;
  const int e = tid % np2, g = tid / np2;
  double s = 0.0;
  if (e < N) {
    // 16 loads in flight, summed in block order
    int b = g;
    for (; b + 15 * G < nb; b += 16 * G) {
      float a[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) a[u] = part[(size_t)(b + u * G) * N + e];
#pragma unroll
      for (int u = 0; u < 16; ++u) s += a[u];
    }
    for (; b < nb; b += G) s += part[(size_t)b * N + e];
  }
  red[tid] = s;
  __syncthreads();
  for (int h = G / 2; h >= 1; h >>= 1) {       // fold the G partial sums of each expert
    if (g < h) red[tid] += red[tid + h * np2];
    __syncthreads();
  }
  if (tid < np2) {
    float t = 0.f;
    if (tid < N) {
      const double P = red[tid] / T;
      const double fe = static_cast<double>(counts[tid]) / (static_cast<double>(T) * k);
      t = static_cast<float>(fe * P);
    }
    term[tid] = t;
  }
  __syncthreads();
  for (int h = np2 / 2; h >= 1; h >>= 1) {
    if (tid < h) term[tid] += term[tid + h];
    __syncthreads();
  }
  if (tid == 0) aux[0] = term[0] * static_cast<float>(N);
}

// Batches of at most 64 tokens (four 16-token partials) in one launch: waves
// 4b .. 4b + 3 of a 1024-thread block compute partial b exactly as block b of
// aux_partial_kernel does, the partials stay in LDS, and the block then runs
// aux_final_kernel's fixed-order folds on them, so the result is bit for bit
// that of the two-launch form.
constexpr int kAuxSmallT = 4 * kAuxTok;
__global__ __launch_bounds__(kAuxFinal) void aux_small_kernel(const float* __restrict__ logits,
                                                              int T, const int32_t* __restrict__ counts,
                                                              int N, int k, float* __restrict__ aux) {
  constexpr int TPW = kAuxTok / 4;
  __shared__ float red[16][256];
  __shared__ float part[4][256];
  __shared__ double fold[kAuxFinal];
  __shared__ float term[256];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nb = (T + kAuxTok - 1) / kAuxTok;
  {
    const int b = w >> 2, wi = w & 3;
    const int tb = b * kAuxTok + wi * TPW;
    float v[TPW][4];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = tb + i;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int e = lane + 64 * c;
        v[i][c] = (t < T && e < N) ? logits[(size_t)t * N + e] : -INFINITY;
      }
    }
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      if (tb + i >= T) break;
      float m = fmaxf(fmaxf(v[i][0], v[i][1]), fmaxf(v[i][2], v[i][3]));
      m = wave_max(m);
      float s = 0.f;
      float p[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        p[c] = (lane + 64 * c < N) ? __expf(v[i][c] - m) : 0.f;
        s += p[c];
      }
      s = wave_sum(s);
      const float inv = 1.f / s;
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] += p[c] * inv;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) red[w][lane + 64 * c] = acc[c];
  }
  __syncthreads();
  for (int i = tid; i < 4 * 256; i += kAuxFinal) {
    const int b = i >> 8, e = i & 255;
    part[b][e] = ((red[4 * b][e] + red[4 * b + 1][e]) + red[4 * b + 2][e]) + red[4 * b + 3][e];
  }
  __syncthreads();
  int np2 = 1;
  while (np2 < N) np2 <<= 1;
  const int G = kAuxFinal / np2;
  const int e = tid % np2, g = tid / np2;
  double s = 0.0;
  if (e < N)
    for (int b = g; b < nb; b += G) s += part[b][e];
  fold[tid] = s;
  __syncthreads();
  for (int h = G / 2; h >= 1; h >>= 1) {
    if (g < h) fold[tid] += fold[tid + h * np2];
    __syncthreads();
  }
  if (tid < np2) {
    float t = 0.f;
    if (tid < N) {
      const double P = fold[tid] / T;
      const double fe = static_cast<double>(counts[tid]) / (static_cast<double>(T) * k);
      t = static_cast<float>(fe * P);
    }
    term[tid] = t;
  }
  __syncthreads();
  for (int h = np2 / 2; h >= 1; h >>= 1) {
    if (tid < h) term[tid] += term[tid + h];
    __syncthreads();
  }
  if (tid == 0) aux[0] = term[0] * static_cast<float>(N);
}

size_t aux_ws_bytes(int T, int N) {
  const size_t nb = (static_cast<size_t>(T) + kAuxTok - 1) / kAuxTok;
  return nb * static_cast<size_t>(N) * sizeof(float);
}

hipError_t launch_aux(const float* logits, const int32_t* counts, int T, int N, int k, float* aux,
                      void* ws, hipStream_t stream) {
  if (T <= kAuxSmallT) {
    hipLaunchKernelGGL(aux_small_kernel, dim3(1), dim3(kAuxFinal), 0, stream, logits, T, counts, N,
                       k, aux);
    return hipGetLastError();
  }
  const int nb = (T + kAuxTok - 1) / kAuxTok;
  float* part = static_cast<float*>(ws);
  hipLaunchKernelGGL(aux_partial_kernel, dim3(nb), dim3(256), 0, stream, logits, T, N, part);
  hipLaunchKernelGGL(aux_final_kernel, dim3(1), dim3(kAuxFinal), 0, stream, part, nb, counts, T, N,
                     k, aux);
  return hipGetLastError();
}

}  // namespace moe
