// Router: logits = hidden . W_router (+ bias), top-k per token, softmax over
// the k selected logits, and the per-expert token histogram.
//
// cf-1.com/news/5914943 §2.1: the router is one small linear layer; the k
// best-scoring experts are kept and their scores softmax-normalised.
// 2kiu.com/news/2885792 §3.1: the logits contract the hidden dimension of the
// tokens with the router weight matrix [hidden, experts].
// 2kiu.com/news/2885792 §5.3: equal logits are ranked by ascending expert id.
// cf-1.com/news/5914943 §2.3: the number of tokens each expert is chosen for.
//
// bf16: 16x16x32 MFMAs; a block's 8 waves split the hidden dimension and
// their partial logits are summed in a fixed order (see router_bf16_kernel).
// fp32: one block = 64 tokens, 4 waves, a plain fp32 dot product per
// (token, expert).  Both end with the same epilogue: the logits tile stays in
// LDS and one wave per token runs k rounds of a wave64 argmax reduction.
#include "common.hpp"
#include "internal.hpp"

namespace moe {

constexpr int kRtTok = 64;        // fp32 router: tokens per block
constexpr int kRtThreads = 256;

__global__ void zero_i32_kernel(int32_t* __restrict__ p, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// Top-k + softmax + histogram of one token, by one wave.  lg: the token's N
// fp32 logits (bias included) in LDS.  Ordering: larger logit first, lower
// expert id first among equal logits.  k rounds of a wave64 argmax.
__device__ __forceinline__ void topk_row(const float* lg, int t, int N, int k,
                                         int32_t* __restrict__ topk_idx,
                                         float* __restrict__ topk_w, int* hist) {
  const int lane = threadIdx.x & 63;
  float v[4];
  unsigned taken = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int e = lane + 64 * c;
    v[c] = (e < N) ? lg[e] : 0.f;
    if (e >= N) taken |= 1u << c;
  }
  float sv[4] = {0.f, 0.f, 0.f, 0.f};
  int si[4] = {0, 0, 0, 0};
  float vmax = 0.f;
  for (int jj = 0; jj < k; ++jj) {
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
    if (jj == 0) vmax = bv;
    if ((jj & 63) == lane) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (c == (jj >> 6)) { sv[c] = bv; si[c] = be; }
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
    const int jj = lane + 64 * c;
    if (jj < k) {
      topk_idx[(size_t)t * k + jj] = si[c];
      topk_w[(size_t)t * k + jj] = __expf(sv[c] - vmax) * inv;
      atomicAdd(&hist[si[c]], 1);
    }
  }
}

// Top-k + softmax + histogram of one token by one thread (k <= kTopkThread):
// k passes over the token's N logits in LDS, pass p taking the best
// (larger logit, then lower expert id) among those ranked after pass p - 1's
// pick.  Many tokens run side by side, one per thread, instead of one token
// per wave through a chain of dependent shuffles.
constexpr int kTopkThread = 16;
__device__ __forceinline__ void topk_thread(const float* lg, int t, int N, int k,
                                            int32_t* __restrict__ topk_idx,
                                            float* __restrict__ topk_w, int* hist) {
  float pv = INFINITY, vmax = 0.f, s = 0.f;
  int pe = -1;
  float sv[kTopkThread];
  int si[kTopkThread];
#pragma unroll
  for (int p = 0; p < kTopkThread; ++p) {
    if (p >= k) break;
    float bv = -INFINITY;
    int be = -1;
    for (int e = 0; e < N; ++e) {
      const float v = lg[e];
      // ranked after the previous pick: smaller logit, or equal logit and larger id
      const bool after = v < pv || (v == pv && e > pe);
      if (after && (be < 0 || v > bv)) {
        bv = v;
        be = e;
      }
    }
    sv[p] = bv;
    si[p] = be;
    pv = bv;
    pe = be;
  }
  vmax = sv[0];
#pragma unroll
  for (int p = 0; p < kTopkThread; ++p)
    if (p < k) s += __expf(sv[p] - vmax);
  const float inv = 1.f / s;
#pragma unroll
  for (int p = 0; p < kTopkThread; ++p) {
    if (p < k) {
      topk_idx[(size_t)t * k + p] = si[p];
      topk_w[(size_t)t * k + p] = __expf(sv[p] - vmax) * inv;
      atomicAdd(&hist[si[p]], 1);
    }
  }
}

// Top-k for the 16 rows of one wave (fp32 router): rows 16w .. 16w+15 of lg.
__device__ __forceinline__ void topk_rows(const float* lg, int ldl, int t0, int T, int N, int k,
                                          int32_t* __restrict__ topk_idx,
                                          float* __restrict__ topk_w, int* hist) {
  const int w = threadIdx.x >> 6;
  for (int rr = 0; rr < 16; ++rr) {
    const int r = w * 16 + rr;
    if (t0 + r >= T) break;
    topk_row(lg + r * ldl, t0 + r, N, k, topk_idx, topk_w, hist);
  }
}

// 8x8 transpose of bf16: r[kk] holds columns 0..7 of k-row kk; c[col] gets
// k-rows 0..7 of column col (an MFMA B operand).
__device__ __forceinline__ void transpose8x8_rt(const uint4 (&r)[8], uint4 (&c)[8]) {
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

// bf16 router.  A block owns 16*MTR tokens; its 8 waves split the k range
// (32-deep steps dealt round-robin) and each wave computes all expert columns
// for all of the block's tokens with 16x16x32 MFMAs:
//   A operand  lane 16g + j: token row j of a 16-token tile, k 8g .. 8g+7
//   B operand  lane 16g + j loads k-rows 8g .. 8g+7 of W_router columns
//              8j .. 8j+7 (+128 per pass) as 16-byte vectors and transposes
//              them in registers; MFMA c then yields column 8j + c.
// The eight partial tiles are summed in wave order through LDS (fixed order,
// so the logits are reproducible), the bias is added, and each wave then runs
// the top-k / softmax / histogram epilogue on its share of the tokens.
// NW = LDS row width (expert columns kept); WAVES * MTR * NW <= 2048 (LDS).
// U = k-steps whose loads are in flight together (register budget permitting).
// With few token tiles the k range is also split across gridDim.y blocks:
// each then writes its partial tile to `part_out` [gridDim.y][T][N] and
// router_finish_kernel completes the tokens.
template <int MTR, int NW, int WAVES, int U>
__global__ __launch_bounds__(64 * WAVES) void router_bf16_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, int T, int d, int N, int k, float* __restrict__ logits,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int32_t* __restrict__ counts,
    float* __restrict__ part_out) {
  constexpr int P = (NW + 127) / 128;          // 128-column passes
  constexpr int ROWS = 16 * MTR;
  constexpr int LD = NW + 1;
  __shared__ float part[WAVES * ROWS * LD];
  __shared__ int hist[256];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15, g = lane >> 4;
  const int t0 = blockIdx.x * ROWS;
  for (int i = tid; i < 256; i += 64 * WAVES) hist[i] = 0;
  // split over k: counts are only added to by router_finish_kernel, which runs
  // after this launch, so one block clears them here
  if (gridDim.y > 1 && blockIdx.x == 0 && blockIdx.y == 0)
    for (int e = tid; e < N; e += 64 * WAVES) counts[e] = 0;

  const uint16_t* arow[MTR];
#pragma unroll
  for (int m = 0; m < MTR; ++m) arow[m] = hidden + (size_t)min(t0 + 16 * m + j, T - 1) * d + 8 * g;
  const bool nvec = (N & 7) == 0;

  f32x4 acc[MTR][P][8];
#pragma unroll
  for (int m = 0; m < MTR; ++m)
#pragma unroll
    for (int q = 0; q < P; ++q)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[m][q][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint4 z4 = make_uint4(0, 0, 0, 0);
  // this block's k range: steps [ks0, ks1) of 32, dealt round-robin to the waves
  const int nks = d / 32;
  const int per = (nks + gridDim.y - 1) / gridDim.y;
  const int ks0 = blockIdx.y * per, ks1 = min(nks, ks0 + per);
  // U k-steps per iteration, all of their loads issued before any MFMA; a step
  // past the end re-reads the last one with a zero A operand (adds nothing)
  for (int ks = ks0 + w; ks < ks1; ks += U * WAVES) {
    uint4 av[U][MTR], wv[U][P][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ksu = ks + u * WAVES;
      const bool live = ksu < ks1;
      const int k0 = 32 * (live ? ksu : ks);
#pragma unroll
      for (int m = 0; m < MTR; ++m)
        av[u][m] = live ? *reinterpret_cast<const uint4*>(arow[m] + k0) : z4;
#pragma unroll
      for (int q = 0; q < P; ++q) {
        const int col = 128 * q + 8 * j;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const uint16_t* src = wr + (size_t)(k0 + 8 * g + kk) * N + col;
          if (nvec) {
            wv[u][q][kk] = (col < N) ? *reinterpret_cast<const uint4*>(src) : z4;
          } else {
            uint32_t e2[4];
#pragma unroll
            for (int c2 = 0; c2 < 4; ++c2) {
              const uint32_t lo = (col + 2 * c2 < N) ? src[2 * c2] : 0u;
              const uint32_t hi = (col + 2 * c2 + 1 < N) ? src[2 * c2 + 1] : 0u;
              e2[c2] = lo | (hi << 16);
            }
            wv[u][q][kk] = make_uint4(e2[0], e2[1], e2[2], e2[3]);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int q = 0; q < P; ++q) {
        uint4 bf[8];
        transpose8x8_rt(wv[u][q], bf);
#pragma unroll
        for (int m = 0; m < MTR; ++m)
#pragma unroll
          for (int c = 0; c < 8; ++c) acc[m][q][c] = mfma16(av[u][m], bf[c], acc[m][q][c]);
      }
  }
  // partial tile of this wave: row 16m + 4g + r, column 128q + 8j + c
  float* mine = part + w * ROWS * LD;
#pragma unroll
  for (int m = 0; m < MTR; ++m)
#pragma unroll
    for (int q = 0; q < P; ++q)
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int col = 128 * q + 8 * j + c;
        if (col < NW) {
#pragma unroll
          for (int r = 0; r < 4; ++r) mine[(16 * m + 4 * g + r) * LD + col] = acc[m][q][c][r];
        }
      }
  __syncthreads();
  // fixed-order sum over the waves; with a k split the block's partial goes out
  if (gridDim.y > 1) {
    float* dst = part_out + (size_t)blockIdx.y * T * N;
    for (int i = tid; i < ROWS * N; i += 64 * WAVES) {
      const int r = i / N, e = i - r * N;
      float v = part[r * LD + e];
#pragma unroll
      for (int ww = 1; ww < WAVES; ++ww) v += part[(ww * ROWS + r) * LD + e];
      if (t0 + r < T) dst[(size_t)(t0 + r) * N + e] = v;
    }
    return;
  }
  // ... else bias, logits out; the sum lands in wave 0's tile
  for (int i = tid; i < ROWS * N; i += 64 * WAVES) {
    const int r = i / N, e = i - r * N;
    float v = part[r * LD + e];
#pragma unroll
    for (int ww = 1; ww < WAVES; ++ww) v += part[(ww * ROWS + r) * LD + e];
    v += (bias != nullptr) ? bias[e] : 0.f;
    part[r * LD + e] = v;
    if (t0 + r < T) logits[(size_t)(t0 + r) * N + e] = v;
  }
  __syncthreads();
  for (int r = w; r < ROWS; r += WAVES) {
    if (t0 + r < T) topk_row(part + r * LD, t0 + r, N, k, topk_idx, topk_w, hist);
  }
  __syncthreads();
  for (int e = tid; e < N; e += 64 * WAVES)
    if (hist[e]) atomicAdd(&counts[e], hist[e]);
}

// ---------------------------------------------------------------- large batches
// For batches of at least kRtBigT tokens the router reads W_router transposed,
// WT [N16][d] (expert rows contiguous in d, rows N .. N16-1 zero), which
// router_prep_kernel writes into the workspace in the same launch that clears
// the counts.  Both MFMA operands are then plain 16-byte loads and a wave keeps
// several 32-deep steps of hidden in flight:
//   16x16x32 MFMAs, A = 16 experts of WT (lane 16g + j: expert 16et + j,
//   k 8g .. 8g+7), B = 16 tokens of hidden (lane 16g + j: token j, the same k).
// A block owns 16 tokens; its waves split d into contiguous ranges, and their
// partial logits are summed in wave order through LDS (fixed order).
constexpr int kRtBigT = 2048;
constexpr int kRtBigWaves = 8;

// Top-k + softmax + histogram of ROWS tokens by the block's 512 threads, LPT =
// 512 / ROWS lanes per token (a power of two, inside one wave): lane s of a
// token holds the logits of experts s, s + LPT, ... (NW / LPT of them, NW = the
// padded expert count), and k rounds each take the best untaken expert, larger
// logit first and lower id among equal ones, by a butterfly over the token's
// lanes.  The token's first lane writes the k picks and their softmax weights.
template <int ROWS, int NW>
__device__ __forceinline__ void topk_lanes(const float* red, int ld, int t0, int nt, int N, int k,
                                           int32_t* __restrict__ topk_idx,
                                           float* __restrict__ topk_w, int* hist) {
  constexpr int LPT = 64 * kRtBigWaves / ROWS;
  constexpr int VPL = NW / LPT > 0 ? NW / LPT : 1;
  const int tid = threadIdx.x;
  const int r = tid / LPT, sl = tid % LPT;
  const bool live = r < nt;
  float v[VPL];
  unsigned taken = 0;
#pragma unroll
  for (int c = 0; c < VPL; ++c) {
    const int e = sl + LPT * c;
    v[c] = (live && e < N) ? red[r * ld + e] : 0.f;
    if (e >= N) taken |= 1u << c;
  }
  float sv[kTopkThread];
  int si[kTopkThread];
#pragma unroll
  for (int jj = 0; jj < kTopkThread; ++jj) {
    if (jj >= k) break;
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int c = 0; c < VPL; ++c) {
      if (!(taken & (1u << c)) && (be == 0x7fffffff || v[c] > bv)) {
        bv = v[c];
        be = sl + LPT * c;
      }
    }
#pragma unroll
    for (int m = 1; m < LPT; m <<= 1) {
      const float ov = __shfl_xor(bv, m, 64);
      const int oe = __shfl_xor(be, m, 64);
      if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
    }
    if (be % LPT == sl) taken |= 1u << (be / LPT);
    sv[jj] = bv;
    si[jj] = be;
  }
  if (live && sl == 0) {
    const float vmax = sv[0];
    float s = 0.f;
#pragma unroll
    for (int jj = 0; jj < kTopkThread; ++jj)
      if (jj < k) s += __expf(sv[jj] - vmax);
    const float inv = 1.f / s;
    const int t = t0 + r;
#pragma unroll
    for (int jj = 0; jj < kTopkThread; ++jj) {
      if (jj < k) {
        topk_idx[(size_t)t * k + jj] = si[jj];
        topk_w[(size_t)t * k + jj] = __expf(sv[jj] - vmax) * inv;
        atomicAdd(&hist[si[jj]], 1);
      }
    }
  }
}

__global__ __launch_bounds__(256) void router_prep_kernel(const uint16_t* __restrict__ wr, int d,
                                                          int N, int N16, uint16_t* __restrict__ wt,
                                                          int32_t* __restrict__ counts) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < N) counts[i] = 0;
  if (i < N16 * d) {
    const int e = i / d, kk = i - e * d;
    wt[i] = e < N ? wr[(size_t)kk * N + e] : (uint16_t)0;
  }
}

template <int MT, int NT>
__global__ __launch_bounds__(64 * kRtBigWaves) __attribute__((amdgpu_waves_per_eu(1, 2)))
void router_wt_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ wt,
    const float* __restrict__ bias, int T, int d, int N, int k, float* __restrict__ logits,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int32_t* __restrict__ counts) {
  constexpr int ROWS = 16 * MT;
  constexpr int LD = 16 * NT + 1;
  // k-steps per batch of loads; two batches are in flight (double buffer of
  // about 96 registers): the next batch is issued before the current one's MFMAs.
  // The 64-token, 64-expert tile takes two steps per batch (128 registers; 60 ->
  // 56 us at 16384 tokens, d 4096) since its accumulators leave room for them.
  constexpr int KB = (MT == 4 && NT == 4) ? 2 : ((48 / (4 * (MT + NT))) < 1 ? 1 : (48 / (4 * (MT + NT))));
  // per-wave partial tiles while they fit in LDS (64 tokens x 64 experts, 32 x 128,
  // 16 x 256); wider tiles add the waves' partials into one tile a wave at a time
  constexpr bool kPerWave = MT * NT <= 16;
  __shared__ float red[kPerWave ? kRtBigWaves : 1][ROWS][LD];
  __shared__ int hist[256];
  __shared__ float sbias[256];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15, g = lane >> 4;
  const int t0 = blockIdx.x * ROWS;
  for (int i = tid; i < 256; i += 64 * kRtBigWaves) hist[i] = 0;
  // the bias is read here, under the k-loop, rather than once per logit in the
  // epilogue (where each read would wait out a memory latency of its own)
  for (int i = tid; i < N; i += 64 * kRtBigWaves) sbias[i] = (bias != nullptr) ? bias[i] : 0.f;

  const int nks = d / 32;
  // k-range q of 8 (q/8 .. (q+1)/8 of d) for this wave; the assignment rotates with
  // the block's place on its XCD (blocks go to the XCDs in turn), so that the
  // XCD's blocks do not all read the same part of WT at the same time.  The
  // partial of range q goes to slot q and the slots are summed in range order,
  // so the sum does not depend on the rotation.
  const int q = (w + (int)(blockIdx.x >> 3)) & (kRtBigWaves - 1);
  const int ks0 = q * nks / kRtBigWaves, ks1 = (q + 1) * nks / kRtBigWaves;
  const uint16_t* brow[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) brow[m] = hidden + (size_t)min(t0 + 16 * m + j, T - 1) * d + 8 * g;
  const uint16_t* arow = wt + (size_t)j * d + 8 * g;
  const size_t tile = (size_t)16 * d;                 // next 16 experts of WT

  f32x4 acc[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int et = 0; et < NT; ++et) acc[m][et] = f32x4{0.f, 0.f, 0.f, 0.f};
  // whole batches of KB steps, double-buffered; the remaining steps one at a time
  uint4 bv[2][KB][MT], av[2][KB][NT];
#define MOE_RT_LOAD(B, NB, K0)                                                              \
  do {                                                                                      \
    _Pragma("unroll") for (int u = 0; u < NB; ++u) {                                        \
      const int k0 = 32 * ((K0) + u);                                                       \
      _Pragma("unroll") for (int m = 0; m < MT; ++m)                                        \
          bv[B][u][m] = *reinterpret_cast<const uint4*>(brow[m] + k0);                      \
      _Pragma("unroll") for (int et = 0; et < NT; ++et)                                     \
          av[B][u][et] = *reinterpret_cast<const uint4*>(arow + et * tile + k0);            \
    }                                                                                       \
  } while (0)
#define MOE_RT_MMA(B, NB)                                                                   \
  do {                                                                                      \
    __builtin_amdgcn_sched_barrier(0); /* loads issued above stay above the MFMAs */        \
    _Pragma("unroll") for (int u = 0; u < NB; ++u)                                          \
        _Pragma("unroll") for (int m = 0; m < MT; ++m)                                      \
            _Pragma("unroll") for (int et = 0; et < NT; ++et)                               \
                acc[m][et] = mfma16(av[B][u][et], bv[B][u][m], acc[m][et]);                 \
  } while (0)
  const int nb = (ks1 - ks0) / KB;
  if (nb > 0) MOE_RT_LOAD(0, KB, ks0);
  int i = 0;
  for (; i + 2 <= nb; i += 2) {
    MOE_RT_LOAD(1, KB, ks0 + (i + 1) * KB);
    MOE_RT_MMA(0, KB);
    if (i + 2 < nb) MOE_RT_LOAD(0, KB, ks0 + (i + 2) * KB);
    MOE_RT_MMA(1, KB);
  }
  if (i < nb) MOE_RT_MMA(0, KB);
  for (int ks = ks0 + nb * KB; ks < ks1; ++ks) {
    MOE_RT_LOAD(0, 1, ks);
    MOE_RT_MMA(0, 1);
  }
#undef MOE_RT_LOAD
#undef MOE_RT_MMA
  // acc[m][et][r]: expert 16 et + 4g + r, token 16 m + j.  Each wave writes its
  // partial logits to the tile of its k-range; one pass then adds the eight tiles
  // in range order (a fixed order, the same sum as adding them one range at a time).
  if (kPerWave) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int et = 0; et < NT; ++et)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          red[kPerWave ? q : 0][16 * m + j][16 * et + 4 * g + r] = acc[m][et][r];
    __syncthreads();
  } else {
    for (int ww = 0; ww < kRtBigWaves; ++ww) {
      if (q == ww) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int et = 0; et < NT; ++et)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              float& dst = red[0][16 * m + j][16 * et + 4 * g + r];
              dst = ww == 0 ? acc[m][et][r] : dst + acc[m][et][r];
            }
      }
      __syncthreads();
    }
  }
  const int nt = min(ROWS, T - t0);
  for (int i = tid; i < ROWS * N; i += 64 * kRtBigWaves) {
    const int r = i / N, e = i - r * N;
    float v = red[0][r][e];
    if (kPerWave) {
#pragma unroll
      for (int ww = 1; ww < kRtBigWaves; ++ww) v += red[kPerWave ? ww : 0][r][e];
    }
    v += sbias[e];
    red[0][r][e] = v;
    if (r < nt) logits[(size_t)(t0 + r) * N + e] = v;
  }
  __syncthreads();
  if (k <= kTopkThread) {
    topk_lanes<ROWS, 16 * NT>(&red[0][0][0], LD, t0, nt, N, k, topk_idx, topk_w, hist);
  } else {
    for (int r = w; r < nt; r += kRtBigWaves)
      topk_row(&red[0][r][0], t0 + r, N, k, topk_idx, topk_w, hist);
  }
  __syncthreads();
  for (int e = tid; e < N; e += 64 * kRtBigWaves)
    if (hist[e]) atomicAdd(&counts[e], hist[e]);
}

// Rows of WT: 16 per expert tile, the tile count rounded up to the kernel's
// power of two (the padding rows are zero).
static int router_n16(int N) {
  int nt = 1;
  while (16 * nt < N) nt <<= 1;
  return 16 * nt;
}

// Completes the tokens of a k-split router: sums the KS partial tiles in
// slice order, adds the bias, writes the logits and runs the top-k epilogue.
// One block = 4 tokens, 4 waves (one token each).
__global__ __launch_bounds__(256) void router_finish_kernel(const float* __restrict__ part, int KS,
                                                            const float* __restrict__ bias, int T,
                                                            int N, int k, float* __restrict__ logits,
                                                            int32_t* __restrict__ topk_idx,
                                                            float* __restrict__ topk_w,
                                                            int32_t* __restrict__ counts) {
  __shared__ float lg[4 * 257];
  __shared__ int hist[256];
  const int tid = threadIdx.x, w = tid >> 6;
  const int t0 = blockIdx.x * 4;
  hist[tid] = 0;
  for (int i = tid; i < 4 * N; i += 256) {
    const int r = i / N, e = i - r * N;
    const int t = t0 + r;
    if (t >= T) continue;
    const float* src = part + (size_t)t * N + e;
    const size_t slice = (size_t)T * N;
    // slices summed in order; their loads are issued 8 at a time
    float v = 0.f;
    int ks = 0;
    for (; ks + 8 <= KS; ks += 8) {
      float a[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) a[u] = src[(ks + u) * slice];
#pragma unroll
      for (int u = 0; u < 8; ++u) v += a[u];
    }
    for (; ks < KS; ++ks) v += src[ks * slice];
    v += (bias != nullptr) ? bias[e] : 0.f;
    lg[r * 257 + e] = v;
    logits[(size_t)t * N + e] = v;
  }
  __syncthreads();
  if (t0 + w < T) topk_row(lg + w * 257, t0 + w, N, k, topk_idx, topk_w, hist);
  __syncthreads();
  for (int e = tid; e < N; e += 256)
    if (hist[e]) atomicAdd(&counts[e], hist[e]);
}

// Number of k slices for the bf16 router: enough blocks to cover the CUs when
// the token tiles alone do not, each slice at least 256 deep.
static int router_kslices(int T, int d, int N) {
  const int rows = (N <= 64) ? (T >= 64 * 256 ? 64 : (T >= 32 * 256 ? 32 : 16))
                             : (N <= 128 ? (T >= 32 * 256 ? 32 : 16) : 16);
  const int tiles = (T + rows - 1) / rows;
  int ks = 256 / tiles;
  ks = ks < 1 ? 1 : ks;
  const int maxks = d / 256 < 1 ? 1 : d / 256;
  return ks > maxks ? maxks : ks;
}

size_t route_ws_bytes(int T, int d, int N) {
  if (T >= kRtBigT) return static_cast<size_t>(router_n16(N)) * d * sizeof(uint16_t);
  const int ks = router_kslices(T, d, N);
  return ks > 1 ? static_cast<size_t>(ks) * T * N * sizeof(float) : 0;
}

// fp32 routers of more than 32 experts (router_f32_wave_kernel below takes the
// rest): 64 tokens per block, the same epilogue after a plain fp32 dot product
// per (token, expert).
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
      // four independent partial sums over q mod 4 (d is a multiple of 64), so that
      // the loads of an unrolled stretch are in flight together instead of one
      // dependent multiply-add at a time (47 -> 36 us for 64 tokens, d 128, 8 experts)
      const float* h = hidden + (size_t)t * d;
      float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
      for (int q = 0; q < d; q += 4)
#pragma unroll
        for (int u = 0; u < 4; ++u) s4[u] = fmaf(h[q + u], wr[(size_t)(q + u) * N + e], s4[u]);
      s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
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

// fp32 router for up to 32 experts: one wave per token, so that a batch of a
// few dozen tokens still spreads over as many CUs and keeps many loads in
// flight (the 64-token-per-block kernel above runs a 64-token batch in one
// block, each thread through chains of dependent loads).  Lane l accumulates
// the token's products for every expert over the hidden positions l, l + 64,
// ... (the loads of U positions issued before their products), the 64 lane sums
// of each expert are added by a butterfly (every lane ends with the same
// bits), and the token's top-k runs on its logits in LDS.
constexpr int kRfWaves = 4, kRfMaxN = 32;
template <int NE>
__global__ __launch_bounds__(64 * kRfWaves) void router_f32_wave_kernel(
    const float* __restrict__ hidden, const float* __restrict__ wr, const float* __restrict__ bias,
    int T, int d, int N, int k, float* __restrict__ logits, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, int32_t* __restrict__ counts) {
  constexpr int U = NE <= 16 ? 4 : 2;
  __shared__ float lg[kRfWaves][NE];
  __shared__ int hist[256];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int t = blockIdx.x * kRfWaves + w;              // wave-uniform
  for (int i = tid; i < 256; i += 64 * kRfWaves) hist[i] = 0;
  if (t < T) {
    float acc[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[e] = 0.f;
    const float* h = hidden + (size_t)t * d;
    int q = lane;                                       // d is a multiple of 64
    for (; q + 64 * (U - 1) < d; q += 64 * U) {
      float hv[U], wv[U][NE];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        hv[u] = h[q + 64 * u];
#pragma unroll
        for (int e = 0; e < NE; ++e) wv[u][e] = e < N ? wr[(size_t)(q + 64 * u) * N + e] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[e] = fmaf(hv[u], wv[u][e], acc[e]);
    }
    for (; q < d; q += 64) {
      const float hv = h[q];
#pragma unroll
      for (int e = 0; e < NE; ++e)
        acc[e] = fmaf(hv, e < N ? wr[(size_t)q * N + e] : 0.f, acc[e]);
    }
    float mine = 0.f;                                   // lane e keeps expert e's logit
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      float v = acc[e];
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
      if (e == lane) mine = v;
    }
    if (lane < N) {
      mine += bias ? bias[lane] : 0.f;
      lg[w][lane] = mine;
      logits[(size_t)t * N + lane] = mine;
    }
  }
  __syncthreads();
  if (t < T) {
    if (k <= kTopkThread) {
      if (lane == 0) topk_thread(lg[w], t, N, k, topk_idx, topk_w, hist);
    } else {
      topk_row(lg[w], t, N, k, topk_idx, topk_w, hist);
    }
  }
  __syncthreads();
  for (int e = tid; e < N; e += 64 * kRfWaves)
    if (hist[e]) atomicAdd(&counts[e], hist[e]);
}

hipError_t launch_route(const void* hidden, const void* w_router, const float* bias, int T, int d,
                        int N, int k, bool bf16, float* logits, int32_t* topk_idx, float* topk_w,
                        int32_t* counts, void* ws, hipStream_t stream) {
  if (bf16 && T >= kRtBigT) {
    const int N16 = router_n16(N);
    uint16_t* wt = static_cast<uint16_t*>(ws);
    const auto* h = static_cast<const uint16_t*>(hidden);
    hipLaunchKernelGGL(router_prep_kernel, dim3((N16 * d + 255) / 256), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(w_router), d, N, N16, wt, counts);
    // about one block per CU: 16 MT tokens per block (MT <= 4, and 1 beyond 128 experts)
    const int mt = T >= 4 * 16 * 256 ? 4 : (T >= 2 * 16 * 256 ? 2 : 1);
    const dim3 block(64 * kRtBigWaves);
#define MOE_ROUTER_WT(MT, NT)                                                                  \
  hipLaunchKernelGGL((router_wt_kernel<MT, NT>), dim3((T + 16 * MT - 1) / (16 * MT)), block, 0,  \
                     stream, h, wt, bias, T, d, N, k, logits, topk_idx, topk_w, counts)
#define MOE_ROUTER_WT_MT(NT)                                                                   \
  do {                                                                                         \
    if (mt == 4) MOE_ROUTER_WT(4, NT);                                                         \
    else if (mt == 2) MOE_ROUTER_WT(2, NT);                                                    \
    else MOE_ROUTER_WT(1, NT);                                                                 \
  } while (0)
    switch (N16 / 16) {
      case 1: MOE_ROUTER_WT_MT(1); break;
      case 2: MOE_ROUTER_WT_MT(2); break;
      case 4: MOE_ROUTER_WT_MT(4); break;
      case 8: MOE_ROUTER_WT_MT(8); break;
      default: MOE_ROUTER_WT(1, 16); break;       // N <= 256
    }
#undef MOE_ROUTER_WT_MT
#undef MOE_ROUTER_WT
    return hipGetLastError();
  }
  const int KS = bf16 ? router_kslices(T, d, N) : 1;
  if (KS == 1)     // otherwise the first router block clears the counts
    hipLaunchKernelGGL(zero_i32_kernel, dim3((N + 255) / 256), dim3(256), 0, stream, counts, N);
  const dim3 grid((T + kRtTok - 1) / kRtTok), block(kRtThreads);
  if (!bf16) {
    const auto* hf = static_cast<const float*>(hidden);
    const auto* wf = static_cast<const float*>(w_router);
    const dim3 gw((T + kRfWaves - 1) / kRfWaves), bw(64 * kRfWaves);
    if (N <= 8)
      hipLaunchKernelGGL(router_f32_wave_kernel<8>, gw, bw, 0, stream, hf, wf, bias, T, d, N, k,
                         logits, topk_idx, topk_w, counts);
    else if (N <= 16)
      hipLaunchKernelGGL(router_f32_wave_kernel<16>, gw, bw, 0, stream, hf, wf, bias, T, d, N, k,
                         logits, topk_idx, topk_w, counts);
    else if (N <= kRfMaxN)
      hipLaunchKernelGGL(router_f32_wave_kernel<32>, gw, bw, 0, stream, hf, wf, bias, T, d, N, k,
                         logits, topk_idx, topk_w, counts);
    else
      hipLaunchKernelGGL(router_f32_kernel, grid, block, 0, stream, hf, wf, bias, T, d, N, k,
                         logits, topk_idx, topk_w, counts);
    return hipGetLastError();
  }
  const auto* h = static_cast<const uint16_t*>(hidden);
  const auto* wr = static_cast<const uint16_t*>(w_router);
  // widest token tile the LDS allows for this N once there are enough tokens
  // for about one block per CU; otherwise split k across blocks as well (KS)
  float* part = static_cast<float*>(ws);
#define MOE_ROUTER(MTR, NW, WV)                                                                \
  hipLaunchKernelGGL((router_bf16_kernel<MTR, NW, WV, 1>),                                   \
                     dim3((T + 16 * MTR - 1) / (16 * MTR), KS), dim3(64 * WV), 0, stream, h,  \
                     wr, bias, T, d, N, k, logits, topk_idx, topk_w, counts, part)
  if (N <= 64) {
    if (T >= 64 * 256) MOE_ROUTER(4, 64, 8);
    else if (T >= 32 * 256) MOE_ROUTER(2, 64, 8);
    else MOE_ROUTER(1, 64, 8);
  } else if (N <= 128) {
    if (T >= 32 * 256) MOE_ROUTER(2, 128, 8);
    else MOE_ROUTER(1, 128, 8);
  } else {
    MOE_ROUTER(1, 256, 8);
  }
  if (KS > 1)
    hipLaunchKernelGGL(router_finish_kernel, dim3((T + 3) / 4), dim3(256), 0, stream, part, KS,
                       bias, T, N, k, logits, topk_idx, topk_w, counts);
#undef MOE_ROUTER
  return hipGetLastError();
}

}  // namespace moe
