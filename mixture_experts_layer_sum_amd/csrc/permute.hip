// Capacity cut and permutation into expert-contiguous rows.
//
// 2kiu.com/news/2885792 §3.1: capacity = int((B*S*k)/E * CF), and each expert
// keeps only its first `capacity` tokens.  cf-1.com/news/5914943 §2.3 (tip):
// tokens over capacity skip the MoE FFN and ride the residual.
// devpress.csdn.net/awstech/6a91abf4... §4.1: scatter the tokens into
// per-expert queues in one vectorised pass instead of a loop over experts.
//
// Deterministic by construction: a token's place at an expert is the number of
// earlier tokens that chose the same expert, computed from per-chunk
// histograms (integer LDS atomics, order-free), a per-expert exclusive scan
// over chunks, and inside a chunk a 256-bit "who chose e" mask per expert
// built with LDS atomic OR (also order-free) and read back with popcounts.
#include "common.hpp"
#include "internal.hpp"

namespace moe {

constexpr int kChunk = 256;   // tokens per chunk = threads per block

// hist[c][e] = number of tokens of chunk c that chose expert e.
__global__ __launch_bounds__(kChunk) void chunk_hist_kernel(const int32_t* __restrict__ topk_idx,
                                                            int T, int N, int k,
                                                            int32_t* __restrict__ hist) {
  __shared__ int h[256];
  const int tid = threadIdx.x, c = blockIdx.x;
  for (int e = tid; e < N; e += kChunk) h[e] = 0;
  __syncthreads();
  const int t = c * kChunk + tid;
  if (t < T)
    for (int j = 0; j < k; ++j) {
      const int e = topk_idx[(size_t)t * k + j];
      if (e >= 0 && e < N) atomicAdd(&h[e], 1);
    }
  __syncthreads();
  for (int e = tid; e < N; e += kChunk) hist[(size_t)c * N + e] = h[e];
}

// One block of 256 threads; thread e scans expert e over the chunks.
__global__ __launch_bounds__(256) void expert_scan_kernel(const int32_t* __restrict__ hist,
                                                          int nchunks, int N, int C,
                                                          int32_t* __restrict__ base,
                                                          int32_t* __restrict__ kept,
                                                          int32_t* __restrict__ offsets) {
  __shared__ int sk[256];
  const int e = threadIdx.x;
  int run = 0;
  if (e < N)
    for (int c = 0; c < nchunks; ++c) {
      base[(size_t)c * N + e] = run;
      run += hist[(size_t)c * N + e];
    }
  const int kp = (e < N) ? (run < C ? run : C) : 0;
  if (e < N) kept[e] = kp;
  sk[e] = kp;
  __syncthreads();
  // inclusive Hillis-Steele scan over 256 entries
  for (int s = 1; s < 256; s <<= 1) {
    const int v = (e >= s) ? sk[e - s] : 0;
    __syncthreads();
    sk[e] += v;
    __syncthreads();
  }
  if (e < N) offsets[e] = sk[e] - kp;
  if (e == N - 1) offsets[N] = sk[e];
}

// Per chunk: place of every (t, j), keep/drop, slot_row and perm_src.
__global__ __launch_bounds__(kChunk) void place_kernel(const int32_t* __restrict__ topk_idx, int T,
                                                       int N, int k, int C,
                                                       const int32_t* __restrict__ base,
                                                       const int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ slot_row,
                                                       int32_t* __restrict__ perm_src) {
  __shared__ unsigned long long mask[256][4];
  __shared__ int off[256];
  __shared__ int bs[256];
  const int tid = threadIdx.x, c = blockIdx.x;
  for (int e = tid; e < N; e += kChunk) {
    mask[e][0] = mask[e][1] = mask[e][2] = mask[e][3] = 0ull;
    off[e] = offsets[e];
    bs[e] = base[(size_t)c * N + e];
  }
  __syncthreads();
  const int t = c * kChunk + tid;
  const int word = tid >> 6;
  const unsigned long long bit = 1ull << (tid & 63);
  if (t < T)
    for (int j = 0; j < k; ++j) {
      const int e = topk_idx[(size_t)t * k + j];
      if (e >= 0 && e < N) atomicOr(&mask[e][word], bit);
    }
  __syncthreads();
  if (t < T)
    for (int j = 0; j < k; ++j) {
      const int e = topk_idx[(size_t)t * k + j];
      int row = -1;
      if (e >= 0 && e < N) {
        int before = 0;
        for (int q = 0; q < word; ++q) before += __popcll(mask[e][q]);
        before += __popcll(mask[e][word] & (bit - 1ull));
        const int place = bs[e] + before;
        if (place < C) {
          row = off[e] + place;
          perm_src[row] = t;
        }
      }
      slot_row[(size_t)t * k + j] = row;
    }
}

// All of the above in one block when every token fits in one chunk (T <= 256,
// decode-sized batches): histogram, capacity, exclusive scan and places.
__global__ __launch_bounds__(kChunk) void permute_one_chunk_kernel(
    const int32_t* __restrict__ topk_idx, int T, int N, int k, int C, int32_t* __restrict__ kept,
    int32_t* __restrict__ offsets, int32_t* __restrict__ slot_row, int32_t* __restrict__ perm_src) {
  __shared__ unsigned long long mask[256][4];
  __shared__ int h[256];
  __shared__ int sk[256];
  __shared__ int off[256];
  const int tid = threadIdx.x;
  mask[tid][0] = mask[tid][1] = mask[tid][2] = mask[tid][3] = 0ull;
  h[tid] = 0;
  __syncthreads();
  const int t = tid;
  const int word = tid >> 6;
  const unsigned long long bit = 1ull << (tid & 63);
  if (t < T)
    for (int j = 0; j < k; ++j) {
      const int e = topk_idx[(size_t)t * k + j];
      if (e >= 0 && e < N) {
        atomicAdd(&h[e], 1);
        atomicOr(&mask[e][word], bit);
      }
    }
  __syncthreads();
  const int e = tid;
  const int kp = (e < N) ? (h[e] < C ? h[e] : C) : 0;
  if (e < N) kept[e] = kp;
  sk[e] = kp;
  __syncthreads();
  for (int s = 1; s < 256; s <<= 1) {     // inclusive Hillis-Steele scan
    const int v = (e >= s) ? sk[e - s] : 0;
    __syncthreads();
    sk[e] += v;
    __syncthreads();
  }
  off[e] = sk[e] - kp;
  if (e < N) offsets[e] = sk[e] - kp;
  if (e == N - 1) offsets[N] = sk[e];
  __syncthreads();
  if (t < T)
    for (int j = 0; j < k; ++j) {
      const int ex = topk_idx[(size_t)t * k + j];
      int row = -1;
      if (ex >= 0 && ex < N) {
        int place = 0;
        for (int q = 0; q < word; ++q) place += __popcll(mask[ex][q]);
        place += __popcll(mask[ex][word] & (bit - 1ull));
        if (place < C) {
          row = off[ex] + place;
          perm_src[row] = t;
        }
      }
      slot_row[(size_t)t * k + j] = row;
    }
}

// Copy hidden[t] into each of its kept rows of x_perm.  One block per token,
// 16-byte vectors; a row is a whole number of vectors.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint4* __restrict__ hidden,
                                                          const int32_t* __restrict__ slot_row,
                                                          int k, int vec_per_row,
                                                          uint4* __restrict__ x_perm) {
  __shared__ int srow[256];
  const int t = blockIdx.x;
  for (int j = threadIdx.x; j < k; j += blockDim.x) srow[j] = slot_row[(size_t)t * k + j];
  __syncthreads();
  const uint4* src = hidden + (size_t)t * vec_per_row;
  for (int v = threadIdx.x; v < vec_per_row; v += blockDim.x) {
    const uint4 x = src[v];
    for (int j = 0; j < k; ++j) {
      const int r = srow[j];
      if (r >= 0) x_perm[(size_t)r * vec_per_row + v] = x;
    }
  }
}

size_t permute_ws_bytes(int T, int N) {
  const size_t nch = (static_cast<size_t>(T) + kChunk - 1) / kChunk;
  return 2 * nch * static_cast<size_t>(N) * sizeof(int32_t);
}

hipError_t launch_permute(const void* hidden, const int32_t* topk_idx, int T, int d, int N, int k,
                          int C, int elem_bytes, void* x_perm, int32_t* perm_src,
                          int32_t* slot_row, int32_t* kept, int32_t* offsets, void* ws,
                          hipStream_t stream) {
  const int nch = (T + kChunk - 1) / kChunk;
  if (nch == 1) {
    hipLaunchKernelGGL(permute_one_chunk_kernel, dim3(1), dim3(kChunk), 0, stream, topk_idx, T, N,
                       k, C, kept, offsets, slot_row, perm_src);
  } else {
    int32_t* hist = static_cast<int32_t*>(ws);
    int32_t* base = hist + static_cast<size_t>(nch) * N;
    hipLaunchKernelGGL(chunk_hist_kernel, dim3(nch), dim3(kChunk), 0, stream, topk_idx, T, N, k,
                       hist);
    hipLaunchKernelGGL(expert_scan_kernel, dim3(1), dim3(256), 0, stream, hist, nch, N, C, base,
                       kept, offsets);
    hipLaunchKernelGGL(place_kernel, dim3(nch), dim3(kChunk), 0, stream, topk_idx, T, N, k, C,
                       base, offsets, slot_row, perm_src);
  }
  const int vpr = (d * elem_bytes) / 16;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(T), dim3(256), 0, stream,
                     static_cast<const uint4*>(hidden), slot_row, k, vpr,
                     static_cast<uint4*>(x_perm));
  return hipGetLastError();
}

}  // namespace moe
