// Grouped expert GEMMs: every expert's SwiGLU FFN over its rows of x_perm.
//
// cf-1.com/news/5914943 §3.3: one grouped GEMM call for all experts instead of
// many small per-expert matmuls.  2kiu.com/news/2885792 §3.3: one kernel for
// all experts, indexed by expert id.  2kiu.com/news/2885792 §5.4: all experts'
// weights live in one tensor sliced by expert id (W1/W3 [N, d, f], W2 [N, f, d]).
// 2kiu.com/news/2885792 §2.2: the experts are SwiGLU FFNs,
//   FFN(x) = (silu(x W1) * (x W3)) W2,  silu(z) = z / (1 + e^-z).
//
// up   : act[r, :] = silu(X[r] W1_e) * (X[r] W3_e)       (SwiGLU fused in the epilogue)
// down : y_perm[r, :] = act[r] W2_e                        (fp32 out)
//
// bf16 path (MFMA): a block computes a 256-row x 256-column tile with 8 waves
// (4 along rows x 2 along columns, 64 x 128 per wave, 16x16x32 bf16 MFMAs,
// fp32 accumulators).  For `up` the 256 columns are 128 columns of W1 and
// the same 128 columns of W3, so the epilogue has both halves of a SwiGLU
// product in the same lane.  k advances 64 at a time through two LDS stages;
// the next stage's global loads are in flight while the current one feeds the
// MFMAs.  The weights are n-contiguous in memory while an MFMA B operand wants
// 8 consecutive k per lane, so every thread loads a 4(k) x 8(n) block and
// transposes it in registers before writing it to LDS k-contiguous.
// The row tiles of all experts are numbered consecutively; a block finds its
// expert with a wave-wide prefix scan of the per-expert tile counts read from
// `offsets` on the device, so the host never needs the routing result.
// Block ids are remapped so that each XCD (blocks are dealt round-robin to the
// 8 XCDs) works on a contiguous range of tiles, grouped 8 row tiles at a time,
// which keeps the A rows and weight columns it streams in its own L2.
#include "common.hpp"
#include "internal.hpp"

namespace moe {

constexpr int kBM = 256, kBN = 256, kBK = 64, kGemmThreads = 512;
constexpr int kLd = kBK + 8;   // bf16 per LDS row (16-byte pad breaks bank aliasing)
constexpr int kGroupM = 8;

// Locate row tile `mt` (tiles of `bm` rows numbered expert by expert).
// Wave-uniform; returns false if mt is past the last tile.  Offsets are
// clamped to [0, max_rows] and made non-decreasing.
__device__ __forceinline__ bool find_tile(const int32_t* __restrict__ offsets, int N, int mt,
                                          int bm, int max_rows, int& e_out, int& r0, int& rend) {
  const int lane = threadIdx.x & 63;
  int before = 0;
  for (int b = 0; b < N; b += 64) {
    const int e = b + lane;
    int o0 = 0, o1 = 0;
    if (e < N) {
      // clamped so that inconsistent offsets can never address rows >= max_rows
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
      const int eo = b + L;
      e_out = eo;
      r0 = __shfl(o0, L, 64) + (mt - before - exc) * bm;
      rend = __shfl(o1, L, 64);
      return true;
    }
    before += total;
  }
  return false;
}

__device__ __forceinline__ void tile_of_block(int mt_bound, int n_tiles, int& mt, int& nt,
                                              bool& valid) {
  const int G = gridDim.x;                 // a multiple of 8
  const int per = G >> 3;
  const int b = blockIdx.x;
  const int logical = (b & 7) * per + (b >> 3);
  const int total = mt_bound * n_tiles;
  valid = logical < total;
  if (!valid) return;
  const int span = kGroupM * n_tiles;
  const int grp = logical / span;
  const int first = grp * kGroupM;
  const int gm = (mt_bound - first) < kGroupM ? (mt_bound - first) : kGroupM;
  const int in = logical - grp * span;
  mt = first + in % gm;
  nt = in / gm;
}

template <bool UP>
__global__ __launch_bounds__(kGemmThreads, 1) void grouped_gemm_bf16_kernel(
    const uint16_t* __restrict__ X, const int32_t* __restrict__ offsets, int N,
    const uint16_t* __restrict__ Wa, const uint16_t* __restrict__ Wb, int K, int Nout,
    int n_tiles, int mt_bound, int max_rows, void* __restrict__ out) {
  __shared__ __align__(16) uint16_t As[2][kBM * kLd];
  __shared__ __align__(16) uint16_t Bs[2][kBN * kLd];

  int mt, nt;
  bool valid;
  tile_of_block(mt_bound, n_tiles, mt, nt, valid);
  if (!valid) return;
  int e, r0, rend;
  if (!find_tile(offsets, N, mt, kBM, max_rows, e, r0, rend)) return;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w & 3, wn = w >> 2;
  const int g = lane >> 4, l16 = lane & 15;
  // UP: block columns [n0, n0+128) of W1 and W3; DOWN: [n0, n0+256) of W2.
  const int n0 = UP ? nt * (kBN / 2) : nt * kBN;

  // ---- global -> register mapping
  // A: 256 rows x 8 chunks of 8 bf16; thread handles items tid + 512*i.
  const uint16_t* a_src[4];
  bool a_ok[4];
  int a_lds[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int item = tid + kGemmThreads * i;
    const int row = item >> 3, ch = item & 7;
    const int gr = r0 + row;
    a_ok[i] = gr < rend;
    a_src[i] = X + (size_t)(a_ok[i] ? gr : r0) * K + 8 * ch;
    a_lds[i] = row * kLd + 8 * ch;
  }
  // B: 4 k-rows x 8 columns per thread.
  const int q = tid & 15;
  int cg, bcol;
  const uint16_t* wbase;
  const size_t wexp = (size_t)e * K * Nout;
  if (UP) {
    cg = (tid >> 4) & 15;
    const bool second = tid >= 256;
    wbase = (second ? Wb : Wa) + wexp + n0 + 8 * cg;
    bcol = (second ? 128 : 0) + 8 * cg;
  } else {
    cg = tid >> 4;  // 0..31
    wbase = Wa + wexp + n0 + 8 * cg;
    bcol = 8 * cg;
  }
  const uint16_t* b_src = wbase + (size_t)(4 * q) * Nout;

  uint4 ra[4], rb[4];
  const uint4 z4 = make_uint4(0, 0, 0, 0);
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ra[i] = a_ok[i] ? *reinterpret_cast<const uint4*>(a_src[i] + k0) : z4;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      rb[r] = *reinterpret_cast<const uint4*>(b_src + (size_t)(k0 + r) * Nout);
  };
  auto lstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(&As[st][a_lds[i]]) = ra[i];
    const uint32_t* r32[4] = {reinterpret_cast<const uint32_t*>(&rb[0]),
                              reinterpret_cast<const uint32_t*>(&rb[1]),
                              reinterpret_cast<const uint32_t*>(&rb[2]),
                              reinterpret_cast<const uint32_t*>(&rb[3])};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int h = c >> 1;
      uint32_t lo, hi;
      if (c & 1) {
        lo = (r32[0][h] >> 16) | (r32[1][h] & 0xFFFF0000u);
        hi = (r32[2][h] >> 16) | (r32[3][h] & 0xFFFF0000u);
      } else {
        lo = (r32[0][h] & 0xFFFFu) | (r32[1][h] << 16);
        hi = (r32[2][h] & 0xFFFFu) | (r32[3][h] << 16);
      }
      *reinterpret_cast<uint2*>(&Bs[st][(bcol + c) * kLd + 4 * q]) = make_uint2(lo, hi);
    }
  };

  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = K / kBK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * kBK);
    const uint16_t* as = As[st];
    const uint16_t* bs = Bs[st];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      uint4 a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const uint4*>(as + (wm * 64 + 16 * i + l16) * kLd + 32 * s + 8 * g);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int col = UP ? ((j < 4) ? (wn * 64 + 16 * j) : (128 + wn * 64 + 16 * (j - 4)))
                           : (wn * 128 + 16 * j);
        const uint4 b = *reinterpret_cast<const uint4*>(bs + (col + l16) * kLd + 32 * s + 8 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i][j] = mfma16(a[i], b, acc[i][j]);
      }
    }
    if (kt + 1 < nk) lstore(st ^ 1);
    __syncthreads();
  }

  // ---- epilogue
  if (UP) {
    uint16_t* act = static_cast<uint16_t*>(out);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = r0 + wm * 64 + 16 * i + 4 * g + r;
        if (row < rend) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float h1 = acc[i][j][r], h3 = acc[i][j + 4][r];
            const float gv = h1 / (1.f + __expf(-h1)) * h3;
            act[(size_t)row * Nout + n0 + wn * 64 + 16 * j + l16] = f32_to_bf16(gv);
          }
        }
      }
  } else {
    float* y = static_cast<float*>(out);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = r0 + wm * 64 + 16 * i + 4 * g + r;
        if (row < rend) {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            y[(size_t)row * Nout + n0 + wn * 128 + 16 * j + l16] = acc[i][j][r];
        }
      }
  }
}

// ---------------------------------------------------------------- fp32 (VALU)
constexpr int kFBM = 64, kFBN = 64, kFBK = 16;

template <bool UP>
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(
    const float* __restrict__ X, const int32_t* __restrict__ offsets, int N,
    const float* __restrict__ Wa, const float* __restrict__ Wb, int K, int Nout, int n_tiles,
    int max_rows, float* __restrict__ out) {
  __shared__ float As[kFBK][kFBM + 1];
  __shared__ float B1[kFBK][kFBN];
  __shared__ float B3[kFBK][kFBN];
  const int mt = blockIdx.x / n_tiles, nt = blockIdx.x % n_tiles;
  int e, r0, rend;
  if (!find_tile(offsets, N, mt, kFBM, max_rows, e, r0, rend)) return;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int n0 = nt * kFBN;
  const size_t wexp = (size_t)e * K * Nout;
  float c1[4][4] = {}, c3[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += kFBK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int item = tid + 256 * i;           // 64 rows x 16 k
      const int row = item >> 4, kk = item & 15;
      const int gr = r0 + row;
      As[kk][row] = gr < rend ? X[(size_t)gr * K + k0 + kk] : 0.f;
      const int kr = item >> 6, col = item & 63;  // 16 k x 64 cols
      B1[kr][col] = Wa[wexp + (size_t)(k0 + kr) * Nout + n0 + col];
      if (UP) B3[kr][col] = Wb[wexp + (size_t)(k0 + kr) * Nout + n0 + col];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kFBK; ++kk) {
      float a[4], b1[4], b3[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        b1[j] = B1[kk][tx * 4 + j];
        if (UP) b3[j] = B3[kk][tx * 4 + j];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          c1[i][j] = fmaf(a[i], b1[j], c1[i][j]);
          if (UP) c3[i][j] = fmaf(a[i], b3[j], c3[i][j]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = r0 + ty * 4 + i;
    if (row >= rend) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      float v = c1[i][j];
      if (UP) v = v / (1.f + expf(-v)) * c3[i][j];
      out[(size_t)row * Nout + col] = v;
    }
  }
}

static int round8(int x) { return (x + 7) & ~7; }

hipError_t launch_expert_up(const void* x_perm, const int32_t* offsets, const void* w1,
                            const void* w3, int N, int d, int f, int max_rows, bool bf16,
                            void* act, hipStream_t stream) {
  if (bf16) {
    const int n_tiles = f / (kBN / 2);
    const int mt_bound = (max_rows + kBM - 1) / kBM + N;
    const int grid = round8(mt_bound * n_tiles);
    hipLaunchKernelGGL(grouped_gemm_bf16_kernel<true>, dim3(grid), dim3(kGemmThreads), 0, stream,
                       static_cast<const uint16_t*>(x_perm), offsets, N,
                       static_cast<const uint16_t*>(w1), static_cast<const uint16_t*>(w3), d, f,
                       n_tiles, mt_bound, max_rows, act);
  } else {
    const int n_tiles = f / kFBN;
    const int mt_bound = (max_rows + kFBM - 1) / kFBM + N;
    hipLaunchKernelGGL(grouped_gemm_f32_kernel<true>, dim3(mt_bound * n_tiles), dim3(256), 0,
                       stream, static_cast<const float*>(x_perm), offsets, N,
                       static_cast<const float*>(w1), static_cast<const float*>(w3), d, f, n_tiles,
                       max_rows, static_cast<float*>(act));
  }
  return hipGetLastError();
}

hipError_t launch_expert_down(const void* act, const int32_t* offsets, const void* w2, int N,
                              int d, int f, int max_rows, bool bf16, float* y_perm,
                              hipStream_t stream) {
  if (bf16) {
    const int n_tiles = d / kBN;
    const int mt_bound = (max_rows + kBM - 1) / kBM + N;
    const int grid = round8(mt_bound * n_tiles);
    hipLaunchKernelGGL(grouped_gemm_bf16_kernel<false>, dim3(grid), dim3(kGemmThreads), 0, stream,
                       static_cast<const uint16_t*>(act), offsets, N,
                       static_cast<const uint16_t*>(w2), static_cast<const uint16_t*>(nullptr), f,
                       d, n_tiles, mt_bound, max_rows, static_cast<void*>(y_perm));
  } else {
    const int n_tiles = d / kFBN;
    const int mt_bound = (max_rows + kFBM - 1) / kFBM + N;
    hipLaunchKernelGGL(grouped_gemm_f32_kernel<false>, dim3(mt_bound * n_tiles), dim3(256), 0,
                       stream, static_cast<const float*>(act), offsets, N,
                       static_cast<const float*>(w2), static_cast<const float*>(nullptr), f, d,
                       n_tiles, max_rows, y_perm);
  }
  return hipGetLastError();
}

}  // namespace moe
