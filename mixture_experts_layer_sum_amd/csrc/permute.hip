// Capacity cut and permutation into expert-contiguous rows.
//
// 2kiu.com/news/2885792 §3.1: an expert's capacity is the floor of the token
// slots (tokens x k) divided by the expert count, times the capacity factor,
// and each expert keeps only its first `capacity` tokens.  cf-1.com/news/5914943 §2.3 (tip):
// tokens over capacity skip the MoE FFN and ride the residual.
// devpress.csdn.net/awstech/6a91abf4... §4.1: scatter the tokens into
// per-expert queues in one vectorised pass instead of a loop over experts.
//
// Deterministic by construction: a token's place at an expert is the number of
// earlier tokens that chose the same expert, computed from per-chunk
// histograms (integer LDS atomics, order-free), a per-expert exclusive scan
// over chunks, and inside a chunk a 256-bit "who chose e" mask per expert
// built with LDS atomic OR (also order-free) and read back with popcounts.
#include <atomic>
#include <mutex>

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

// Exclusive scan of expert e's counts over the chunks, in chunk order:
// base[c][e] = sum of hist[c'][e] for c' < c; returns the total.  The loads
// are issued 16 at a time (they do not depend on each other), so a thread
// waits on memory about nchunks / 16 times instead of nchunks times.
__device__ __forceinline__ int scan_chunks(const int32_t* __restrict__ hist, int nchunks, int N,
                                           int e, int32_t* __restrict__ base) {
  int run = 0, c = 0;
  for (; c + 16 <= nchunks; c += 16) {
    int v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = hist[(size_t)(c + u) * N + e];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      base[(size_t)(c + u) * N + e] = run;
      run += v[u];
    }
  }
  for (; c < nchunks; ++c) {
    base[(size_t)c * N + e] = run;
    run += hist[(size_t)c * N + e];
  }
  return run;
}

// One block of 256 threads; thread e scans expert e over the chunks.
__global__ __launch_bounds__(256) void expert_scan_kernel(const int32_t* __restrict__ hist,
                                                          int nchunks, int N, int C,
                                                          int32_t* __restrict__ base,
                                                          int32_t* __restrict__ kept,
                                                          int32_t* __restrict__ offsets) {
  __shared__ int sk[256];
  const int e = threadIdx.x;
  const int run = (e < N) ? scan_chunks(hist, nchunks, N, e, base) : 0;
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

// All of the above, and the copy of the rows, in one launch when every token
// fits in one chunk (T <= 256, decode-sized batches).  Block t (one per token)
// builds the whole chunk's histogram, capacity cut, exclusive scan and
// per-expert masks in LDS (the same values in every block: the inputs are a
// few KB and the work is integer and order-free), then places its own token's
// slots and copies its hidden row into them; block 0 also writes kept and
// offsets.  One launch instead of a dispatch block followed by a copy grid.
__global__ __launch_bounds__(kChunk) void permute_one_chunk_kernel(
    const int32_t* __restrict__ topk_idx, int T, int N, int k, int C, int32_t* __restrict__ kept,
    int32_t* __restrict__ offsets, int32_t* __restrict__ slot_row, int32_t* __restrict__ perm_src,
    const uint4* __restrict__ hidden, int vec_per_row, uint4* __restrict__ x_perm) {
  __shared__ unsigned long long mask[256][4];
  __shared__ int h[256];
  __shared__ int sk[256];
  __shared__ int off[256];
  __shared__ int srow[256];
  const int tid = threadIdx.x;
  mask[tid][0] = mask[tid][1] = mask[tid][2] = mask[tid][3] = 0ull;
  h[tid] = 0;
  __syncthreads();
  {
    const int t = tid;
    const int word = t >> 6;
    const unsigned long long bit = 1ull << (t & 63);
    if (t < T)
      for (int j = 0; j < k; ++j) {
        const int e = topk_idx[(size_t)t * k + j];
        if (e >= 0 && e < N) {
          atomicAdd(&h[e], 1);
          atomicOr(&mask[e][word], bit);
        }
      }
  }
  __syncthreads();
  const int e = tid;
  const int kp = (e < N) ? (h[e] < C ? h[e] : C) : 0;
  sk[e] = kp;
  __syncthreads();
  for (int s = 1; s < 256; s <<= 1) {     // inclusive Hillis-Steele scan
    const int v = (e >= s) ? sk[e - s] : 0;
    __syncthreads();
    sk[e] += v;
    __syncthreads();
  }
  off[e] = sk[e] - kp;
  if (blockIdx.x == 0) {
    if (e < N) {
      kept[e] = kp;
      offsets[e] = sk[e] - kp;
    }
    if (e == N - 1) offsets[N] = sk[e];
  }
  __syncthreads();
  // this block's token: its slots' rows
  const int t = blockIdx.x;
  const int word = t >> 6;
  const unsigned long long bit = 1ull << (t & 63);
  for (int j = tid; j < k; j += kChunk) {
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
    if (j < 256) srow[j] = row;
  }
  __syncthreads();
  const int kk = k < 256 ? k : 256;
  bool kept_any = false;
  for (int j = 0; j < kk; ++j) kept_any |= srow[j] >= 0;
  if (!kept_any) return;
  const uint4* src = hidden + (size_t)t * vec_per_row;
  for (int v = tid; v < vec_per_row; v += kChunk) {
    const uint4 x = src[v];
    for (int j = 0; j < kk; ++j) {
      const int r = srow[j];
      if (r >= 0) x_perm[(size_t)r * vec_per_row + v] = x;
    }
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
  // a token whose every slot was dropped is not read at all (block-uniform)
  bool kept_any = false;
  for (int j = 0; j < k; ++j) kept_any |= srow[j] >= 0;
  if (!kept_any) return;
  const uint4* src = hidden + (size_t)t * vec_per_row;
  for (int v = threadIdx.x; v < vec_per_row; v += blockDim.x) {
    const uint4 x = src[v];
    for (int j = 0; j < k; ++j) {
      const int r = srow[j];
      if (r >= 0) x_perm[(size_t)r * vec_per_row + v] = x;
    }
  }
}

// ---------------------------------------------------------------- overflow re-routing
// hotelren.com/news/3071227 §4.2 (capacity-aware routing: mask the original
// pick of an over-capacity token and take its next-best expert),
// 2kiu.com/news/2885792 §2.2 and hotelren.com/news/3071227 §2.2 (tokens over
// capacity are dropped or sent to the next-best expert),
// devpress.csdn.net/awstech/6a91abf4... §2.3 (overflow goes to idle experts).
// One second dispatch round after the capacity cut: each dropped assignment,
// in slot order within its token, proposes the highest-logit expert that is
// not one of the token's picks, not proposed by an earlier dropped slot of
// the token, and had room after the first round; experts admit proposals in
// token order up to the room left.  Both rounds use the same order-free
// machinery as the first (chunk histograms, per-expert scan, bitmask ranks).

// rank[s] = place of slot s at expert ids[s] in token order (base[c][e] +
// earlier slots of the chunk), or -1 where ids[s] is not an expert.
__global__ __launch_bounds__(kChunk) void rank_kernel(const int32_t* __restrict__ ids, int T,
                                                      int N, int k,
                                                      const int32_t* __restrict__ base,
                                                      int32_t* __restrict__ rank) {
  __shared__ unsigned long long mask[256][4];
  __shared__ int bs[256];
  const int tid = threadIdx.x, c = blockIdx.x;
  for (int e = tid; e < N; e += kChunk) {
    mask[e][0] = mask[e][1] = mask[e][2] = mask[e][3] = 0ull;
    bs[e] = base[(size_t)c * N + e];
  }
  __syncthreads();
  const int t = c * kChunk + tid;
  const int word = tid >> 6;
  const unsigned long long bit = 1ull << (tid & 63);
  if (t < T)
    for (int j = 0; j < k; ++j) {
      const int e = ids[(size_t)t * k + j];
      if (e >= 0 && e < N) atomicOr(&mask[e][word], bit);
    }
  __syncthreads();
  if (t < T)
    for (int j = 0; j < k; ++j) {
      const int e = ids[(size_t)t * k + j];
      int r = -1;
      if (e >= 0 && e < N) {
        r = bs[e];
        for (int q = 0; q < word; ++q) r += __popcll(mask[e][q]);
        r += __popcll(mask[e][word] & (bit - 1ull));
      }
      rank[(size_t)t * k + j] = r;
    }
}

// First-round totals: kept1[e] = min(count_e, C).
__global__ __launch_bounds__(256) void first_round_scan_kernel(const int32_t* __restrict__ hist,
                                                               int nchunks, int N, int C,
                                                               int32_t* __restrict__ base,
                                                               int32_t* __restrict__ kept1) {
  const int e = threadIdx.x;
  if (e >= N) return;
  const int run = scan_chunks(hist, nchunks, N, e, base);
  kept1[e] = run < C ? run : C;
}

// One wave per token: proposals of its dropped slots.  The token's logits row
// is read once (coalesced; fp32, the precision the router produced it in), lane
// l holding experts l, l + 64, ...; each dropped slot, in slot order, takes the
// expert with room that the token does not hold yet with the highest logit,
// ties to the lower expert id (a wave-wide argmax over (logit, -id)).
constexpr int kProposeWaves = 4;
__global__ __launch_bounds__(64 * kProposeWaves) void propose_kernel(
    const int32_t* __restrict__ topk_idx, const float* __restrict__ logits,
    const int32_t* __restrict__ rank1, const int32_t* __restrict__ kept1, int T, int N, int k,
    int C, int32_t* __restrict__ prop) {
  __shared__ int room[256];
  for (int e = threadIdx.x; e < 256; e += blockDim.x) room[e] = (e < N) && kept1[e] < C;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kProposeWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  // bit c of `ok`: expert lane + 64 c is still a candidate (a mask rather than an
  // array, which the dynamic index below would put in scratch memory)
  float v[4];
  unsigned ok = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int e = lane + 64 * c;
    if (e < N && room[e]) ok |= 1u << c;
    v[c] = e < N ? logits[(size_t)t * N + e] : 0.f;
  }
  for (int j = 0; j < k; ++j) {                  // the token's own experts are not candidates
    const int e = topk_idx[(size_t)t * k + j];
    if (e >= 0 && e < N && (e & 63) == lane) ok &= ~(1u << (e >> 6));
  }
  for (int j = 0; j < k; ++j) {
    const size_t s = (size_t)t * k + j;
    const int e0 = topk_idx[s];
    int best = -1;
    if (e0 >= 0 && e0 < N && rank1[s] >= C) {   // the same for the whole wave
      float bv = 0.f;
      int be = 0x7FFFFFFF;                       // no candidate
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (((ok >> c) & 1u) && (be == 0x7FFFFFFF || v[c] > bv)) {
          bv = v[c];
          be = lane + 64 * c;
        }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        const float ov = __shfl_xor(bv, m, 64);
        const int oe = __shfl_xor(be, m, 64);
        const bool take = oe != 0x7FFFFFFF &&
                          (be == 0x7FFFFFFF || ov > bv || (ov == bv && oe < be));
        if (take) {
          bv = ov;
          be = oe;
        }
      }
      if (be != 0x7FFFFFFF) {
        best = be;
        if ((be & 63) == lane) ok &= ~(1u << (be >> 6));
      }
    }
    if (lane == 0) prop[s] = best;
  }
}

// Second-round totals and the final layout: kept2[e] = min(proposals_e,
// C - kept1[e]); kept = kept1 + kept2; offsets = exclusive scan of kept.
__global__ __launch_bounds__(256) void second_round_scan_kernel(const int32_t* __restrict__ hist2,
                                                                int nchunks, int N, int C,
                                                                const int32_t* __restrict__ kept1,
                                                                int32_t* __restrict__ base2,
                                                                int32_t* __restrict__ kept,
                                                                int32_t* __restrict__ offsets) {
  __shared__ int sk[256];
  const int e = threadIdx.x;
  const int run = (e < N) ? scan_chunks(hist2, nchunks, N, e, base2) : 0;
  int kp = 0;
  if (e < N) {
    const int k1 = kept1[e];
    const int r2 = C - k1;
    kp = k1 + (run < r2 ? run : r2);
    kept[e] = kp;
  }
  sk[e] = kp;
  __syncthreads();
  for (int s = 1; s < 256; s <<= 1) {     // inclusive Hillis-Steele scan
    const int v = (e >= s) ? sk[e - s] : 0;
    __syncthreads();
    sk[e] += v;
    __syncthreads();
  }
  if (e < N) offsets[e] = sk[e] - kp;
  if (e == N - 1) offsets[N] = sk[e];
}

// Rows of both rounds: first-round places first inside an expert, then the
// admitted second-round places.
__global__ __launch_bounds__(256) void reroute_place_kernel(
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ rank1,
    const int32_t* __restrict__ prop, const int32_t* __restrict__ rank2,
    const int32_t* __restrict__ kept1, const int32_t* __restrict__ offsets, int T, int N, int k,
    int C, int32_t* __restrict__ slot_row, int32_t* __restrict__ perm_src) {
  const size_t s = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= (size_t)T * k) return;
  const int t = (int)(s / k);
  const int e1 = topk_idx[s];
  int row = -1;
  if (e1 >= 0 && e1 < N && rank1[s] < C) {
    row = offsets[e1] + rank1[s];
  } else {
    const int e2 = prop[s];
    if (e2 >= 0 && rank2[s] < C - kept1[e2]) row = offsets[e2] + kept1[e2] + rank2[s];
  }
  slot_row[s] = row;
  if (row >= 0) perm_src[row] = t;
}

size_t permute_reroute_ws_bytes(int T, int N, int k) {
  const size_t nch = (static_cast<size_t>(T) + kChunk - 1) / kChunk;
  const size_t ints = 4 * nch * N + N + 3 * static_cast<size_t>(T) * k;
  return ints * sizeof(int32_t);
}

hipError_t launch_permute_reroute(const void* hidden, const int32_t* topk_idx,
                                  const float* logits, int T, int d, int N, int k, int C,
                                  int elem_bytes, void* x_perm, int32_t* perm_src,
                                  int32_t* slot_row, int32_t* kept, int32_t* offsets, void* ws,
                                  hipStream_t stream) {
  const int nch = (T + kChunk - 1) / kChunk;
  const size_t tk = static_cast<size_t>(T) * k;
  int32_t* hist1 = static_cast<int32_t*>(ws);
  int32_t* base1 = hist1 + static_cast<size_t>(nch) * N;
  int32_t* hist2 = base1 + static_cast<size_t>(nch) * N;
  int32_t* base2 = hist2 + static_cast<size_t>(nch) * N;
  int32_t* kept1 = base2 + static_cast<size_t>(nch) * N;
  int32_t* rank1 = kept1 + N;
  int32_t* prop = rank1 + tk;
  int32_t* rank2 = prop + tk;
  hipLaunchKernelGGL(chunk_hist_kernel, dim3(nch), dim3(kChunk), 0, stream, topk_idx, T, N, k,
                     hist1);
  hipLaunchKernelGGL(first_round_scan_kernel, dim3(1), dim3(256), 0, stream, hist1, nch, N, C,
                     base1, kept1);
  hipLaunchKernelGGL(rank_kernel, dim3(nch), dim3(kChunk), 0, stream, topk_idx, T, N, k, base1,
                     rank1);
  hipLaunchKernelGGL(propose_kernel, dim3((T + kProposeWaves - 1) / kProposeWaves),
                     dim3(64 * kProposeWaves), 0, stream, topk_idx, logits, rank1, kept1, T, N, k,
                     C, prop);
  hipLaunchKernelGGL(chunk_hist_kernel, dim3(nch), dim3(kChunk), 0, stream, prop, T, N, k, hist2);
  hipLaunchKernelGGL(second_round_scan_kernel, dim3(1), dim3(256), 0, stream, hist2, nch, N, C,
                     kept1, base2, kept, offsets);
  hipLaunchKernelGGL(rank_kernel, dim3(nch), dim3(kChunk), 0, stream, prop, T, N, k, base2,
                     rank2);
  hipLaunchKernelGGL(reroute_place_kernel, dim3((unsigned)((tk + 255) / 256)), dim3(256), 0,
                     stream, topk_idx, rank1, prop, rank2, kept1, offsets, T, N, k, C, slot_row,
                     perm_src);
  const int vpr = (d * elem_bytes) / 16;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(T), dim3(256), 0, stream,
                     static_cast<const uint4*>(hidden), slot_row, k, vpr,
                     static_cast<uint4*>(x_perm));
  return hipGetLastError();
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
  const int vpr = (d * elem_bytes) / 16;
  if (nch == 1) {
    if (T == 0) return hipGetLastError();
    hipLaunchKernelGGL(permute_one_chunk_kernel, dim3(T), dim3(kChunk), 0, stream, topk_idx, T, N,
                       k, C, kept, offsets, slot_row, perm_src, static_cast<const uint4*>(hidden),
                       vpr, static_cast<uint4*>(x_perm));
    return hipGetLastError();
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
  hipLaunchKernelGGL(gather_rows_kernel, dim3(T), dim3(256), 0, stream,
                     static_cast<const uint4*>(hidden), slot_row, k, vpr,
                     static_cast<uint4*>(x_perm));
  return hipGetLastError();
}

// ---------------------------------------------------------------- no-allocation variant
// moe_permute_noalloc runs the kernels above with the chunk tables in a
// file-scope device array instead of a caller workspace, for callers that
// cannot allocate.  Each device holds its own copy of the array from the
// library's load until the process ends; calls that overlap on one device
// share it and race.  Nothing in it needs clearing: chunk_hist_kernel writes
// every entry of the histogram table and expert_scan_kernel every entry of
// the base table before either is read.
static __device__ __align__(256) int32_t scratch[kPermuteNoAllocScratchBytes / sizeof(int32_t)];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<int32_t*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's address of `scratch` (the host-side name is only a
// stand-in: passing it to a kernel would fault).  Looked up once per device,
// with that device current, and kept.
hipError_t scratch_of_current_device(int32_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  int32_t* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      void* q = nullptr;
      e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (q == nullptr) return hipErrorInvalidSymbol;
      p = static_cast<int32_t*>(q);
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}
}  // namespace

hipError_t launch_permute_noalloc(const void* hidden, const int32_t* topk_idx, int T, int d, int N,
                                  int k, int C, int elem_bytes, void* x_perm, int32_t* perm_src,
                                  int32_t* slot_row, int32_t* kept, int32_t* offsets,
                                  hipStream_t stream) {
  int32_t* ws = nullptr;
  const hipError_t e = scratch_of_current_device(&ws);
  if (e != hipSuccess) return e;
  return launch_permute(hidden, topk_idx, T, d, N, k, C, elem_bytes, x_perm, perm_src, slot_row,
                        kept, offsets, ws, stream);
}

}  // namespace moe
