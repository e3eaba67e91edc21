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

constexpr int kBM = 256, kBN = 256, kBK = 64, kGemmThreads = 256;
constexpr int kLd = kBK + 8;   // bf16 per LDS row (16-byte pad breaks bank aliasing)
constexpr int kGroupM = 8;

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(const uint4& a, const uint4& b, f32x16 acc) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
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

// Block -> (row tile, column tile).  Blocks are dealt round-robin to the 8
// XCDs, so block b runs on XCD b % 8: give XCD x the contiguous range
// [x*per, (x+1)*per) of the real tiles (per = ceil(tiles / 8)), and inside a
// range walk kGroupM row tiles for every column tile, so the blocks an XCD
// runs at the same time share A rows and weight columns in its L2.
__device__ __forceinline__ bool tile_of_block(int m_tiles, int n_tiles, int& mt, int& nt) {
  const int total = m_tiles * n_tiles;
  const int per = (total + 7) >> 3;
  const int b = blockIdx.x;
  const int local = b >> 3;
  if (local >= per) return false;
  const int logical = (b & 7) * per + local;
  if (logical >= total) return false;
  const int span = kGroupM * n_tiles;
  const int grp = logical / span;
  const int first = grp * kGroupM;
  const int gm = (m_tiles - first) < kGroupM ? (m_tiles - first) : kGroupM;
  const int in = logical - grp * span;
  mt = first + in % gm;
  nt = in / gm;
  return true;
}

typedef int i32x4 __attribute__((ext_vector_type(4)));
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9 family)

__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// Transpose a 4(k) x 8(n) block of bf16 held as four 8-wide rows into eight
// 4-wide columns (two packed dwords each) and store them k-contiguous in LDS.
__device__ __forceinline__ void store_kmajor(uint16_t* dst, int ld, const uint4& r0,
                                             const uint4& r1, const uint4& r2, const uint4& r3) {
  const uint32_t a[4] = {r0.x, r0.y, r0.z, r0.w};
  const uint32_t b[4] = {r1.x, r1.y, r1.z, r1.w};
  const uint32_t c[4] = {r2.x, r2.y, r2.z, r2.w};
  const uint32_t d[4] = {r3.x, r3.y, r3.z, r3.w};
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint2 even = make_uint2((a[m] & 0xFFFFu) | (b[m] << 16), (c[m] & 0xFFFFu) | (d[m] << 16));
    const uint2 odd = make_uint2((a[m] >> 16) | (b[m] & 0xFFFF0000u), (c[m] >> 16) | (d[m] & 0xFFFF0000u));
    *reinterpret_cast<uint2*>(dst + (2 * m) * ld) = even;
    *reinterpret_cast<uint2*>(dst + (2 * m + 1) * ld) = odd;
  }
}

// 256 x 256 block tile, 4 waves in 2 x 2, 128 x 128 per wave on 32x32x16 bf16
// MFMAs (4 x 4 accumulators of 16 floats per lane, held in AGPRs).
// Operand convention: lane l holds row/column (l % 32) and k values
// 8*(l/32) .. 8*(l/32)+7 of a 16-deep k slice, for A and B alike.
// Result: lane l, element r is D[8*(r/4) + 4*(l/32) + r%4][l % 32].
// Global loads are raw buffer loads: rows past the tile's last valid row fall
// outside the A descriptor's range and read as zero.
template <bool UP>
__global__ __launch_bounds__(kGemmThreads, 1) void grouped_gemm_bf16_kernel(
    const uint16_t* __restrict__ X, const int32_t* __restrict__ offsets, int N,
    const uint16_t* __restrict__ Wa, const uint16_t* __restrict__ Wb, int K, int Nout,
    int n_tiles, int max_rows, void* __restrict__ out) {
  __shared__ __align__(16) uint16_t As[2][kBM * kLd];
  __shared__ __align__(16) uint16_t Bs[2][kBN * kLd];

  const int m_tiles = count_tiles(offsets, N, kBM, max_rows);
  int mt, nt;
  if (!tile_of_block(m_tiles, n_tiles, mt, nt)) return;
  int e, r0, rend;
  if (!find_tile(offsets, N, mt, kBM, max_rows, e, r0, rend)) return;
  // the tile coordinates are block-uniform: keep them (and the descriptors
  // built from them) in scalar registers
  e = __builtin_amdgcn_readfirstlane(e);
  r0 = __builtin_amdgcn_readfirstlane(r0);
  rend = __builtin_amdgcn_readfirstlane(rend);
  nt = __builtin_amdgcn_readfirstlane(nt);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w & 1, wn = w >> 1;
  const int l32 = lane & 31, h = lane >> 5;
  // UP: block columns [n0, n0+128) of W1 and of W3; DOWN: [n0, n0+256) of W2.
  const int n0 = UP ? nt * (kBN / 2) : nt * kBN;

  const int tile_rows = min(rend - r0, kBM);
  const __amdgpu_buffer_rsrc_t a_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(X + (size_t)r0 * K), 0, tile_rows * K * 2, kRsrcWord3);
  const size_t wexp = (size_t)e * K * Nout;
  const int wbytes = K * Nout * 2;
  const __amdgpu_buffer_rsrc_t b_rs0 =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Wa + wexp), 0, wbytes, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t b_rs1 = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>((UP ? Wb : Wa) + wexp), 0, wbytes, kRsrcWord3);

  // A: 256 rows x 8 chunks of 8 bf16 = 2048 items; item tid + 256*i is row
  // (tid/8) + 32*i, chunk tid%8.
  const uint32_t a_voff = (uint32_t)(((tid >> 3) * K + 8 * (tid & 7)) * 2);
  const uint32_t a_step = (uint32_t)(32 * K * 2);
  const int a_lds = (tid >> 3) * kLd + 8 * (tid & 7);
  // B: two 4(k) x 8(n) blocks per thread; q = k quad, cg = column group.
  const int q = tid & 15;
  const int cg0 = tid >> 4;
  const int cg1 = UP ? cg0 : cg0 + 16;
  const uint32_t b_voff0 = (uint32_t)(((4 * q) * Nout + n0 + 8 * cg0) * 2);
  const uint32_t b_voff1 = (uint32_t)(((4 * q) * Nout + n0 + 8 * cg1) * 2);
  const uint32_t b_row = (uint32_t)(Nout * 2);
  const int bcol0 = 8 * cg0;
  const int bcol1 = UP ? 128 + 8 * cg0 : 8 * cg1;

  // Two register sets of one k-step each: the loads for step kt+2 are issued
  // at the top of step kt and written to LDS in the middle of step kt+1, so
  // they have about one and a half k-steps of MFMA work to arrive.
#define MOE_REGSET(P)                                                   \
  uint4 P##a0, P##a1, P##a2, P##a3, P##a4, P##a5, P##a6, P##a7;         \
  uint4 P##b00, P##b01, P##b02, P##b03, P##b10, P##b11, P##b12, P##b13
  MOE_REGSET(x);
  MOE_REGSET(y);
#undef MOE_REGSET

#define MOE_GLOAD(P, k0)                                                \
  do {                                                                  \
    const uint32_t ks = (uint32_t)(k0) * 2;                             \
    const uint32_t kb = (uint32_t)(k0) * b_row;                         \
    P##a0 = bload(a_rs, a_voff, ks);                                    \
    P##a1 = bload(a_rs, a_voff + a_step, ks);                           \
    P##a2 = bload(a_rs, a_voff + 2 * a_step, ks);                       \
    P##a3 = bload(a_rs, a_voff + 3 * a_step, ks);                       \
    P##a4 = bload(a_rs, a_voff + 4 * a_step, ks);                       \
    P##a5 = bload(a_rs, a_voff + 5 * a_step, ks);                       \
    P##a6 = bload(a_rs, a_voff + 6 * a_step, ks);                       \
    P##a7 = bload(a_rs, a_voff + 7 * a_step, ks);                       \
    P##b00 = bload(b_rs0, b_voff0, kb);                                 \
    P##b01 = bload(b_rs0, b_voff0 + b_row, kb);                         \
    P##b02 = bload(b_rs0, b_voff0 + 2 * b_row, kb);                     \
    P##b03 = bload(b_rs0, b_voff0 + 3 * b_row, kb);                     \
    P##b10 = bload(b_rs1, b_voff1, kb);                                 \
    P##b11 = bload(b_rs1, b_voff1 + b_row, kb);                         \
    P##b12 = bload(b_rs1, b_voff1 + 2 * b_row, kb);                     \
    P##b13 = bload(b_rs1, b_voff1 + 3 * b_row, kb);                     \
  } while (0)

#define MOE_LSTORE(P, st)                                               \
  do {                                                                  \
    uint16_t* as_ = As[st] + a_lds;                                     \
    *reinterpret_cast<uint4*>(as_) = P##a0;                             \
    *reinterpret_cast<uint4*>(as_ + 32 * kLd) = P##a1;                  \
    *reinterpret_cast<uint4*>(as_ + 64 * kLd) = P##a2;                  \
    *reinterpret_cast<uint4*>(as_ + 96 * kLd) = P##a3;                  \
    *reinterpret_cast<uint4*>(as_ + 128 * kLd) = P##a4;                 \
    *reinterpret_cast<uint4*>(as_ + 160 * kLd) = P##a5;                 \
    *reinterpret_cast<uint4*>(as_ + 192 * kLd) = P##a6;                 \
    *reinterpret_cast<uint4*>(as_ + 224 * kLd) = P##a7;                 \
    store_kmajor(Bs[st] + bcol0 * kLd + 4 * q, kLd, P##b00, P##b01, P##b02, P##b03); \
    store_kmajor(Bs[st] + bcol1 * kLd + 4 * q, kLd, P##b10, P##b11, P##b12, P##b13); \
  } while (0)

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // this wave's rows / columns inside the block tile (LDS element offsets)
  const int a_frag = (wm * 128 + l32) * kLd + 8 * h;
  int b_frag[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = UP ? ((j < 2) ? (wn * 64 + 32 * j) : (128 + wn * 64 + 32 * (j - 2)))
                       : (wn * 128 + 32 * j);
    b_frag[j] = (col + l32) * kLd + 8 * h;
  }

  // Fragment registers, double-buffered: sub-step s+1's fragments are read
  // from LDS while sub-step s's MFMAs run.
  uint4 fa0[4], fb0[4], fa1[4], fb1[4];
#define MOE_LOADF(F, st, s)                                                                  \
  do {                                                                                      \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                           \
        fa##F[i] = *reinterpret_cast<const uint4*>(As[st] + a_frag + 32 * i * kLd + 16 * (s)); \
    _Pragma("unroll") for (int j = 0; j < 4; ++j)                                           \
        fb##F[j] = *reinterpret_cast<const uint4*>(Bs[st] + b_frag[j] + 16 * (s));          \
  } while (0)
#define MOE_MMA(F)                                                                           \
  do {                                                                                      \
    _Pragma("unroll") for (int i = 0; i < 4; ++i)                                           \
        _Pragma("unroll") for (int j = 0; j < 4; ++j)                                       \
            acc[i][j] = mfma32(fa##F[i], fb##F[j], acc[i][j]);                              \
  } while (0)
#define MOE_FENCE() __builtin_amdgcn_sched_barrier(0)

  // One k-step reading LDS stage `st` (four 16-deep sub-steps).  Loads for
  // step kt+2 go to register set L at the top; set S (step kt+1) is written to
  // the other stage in the second sub-step; the barrier sits before the last
  // sub-step's MFMAs so that the next stage's first fragments are read while
  // they run.  The body has no branches (past the end, loads repeat the last
  // k-step and the extra LDS writes and reads are never used), so the
  // hardware wait counters only ever wait for the loads a step consumes.
  // Interleaving hints for the scheduler (groups are emitted in this order):
  // 0x008 MFMA, 0x020 VMEM read, 0x100 LDS read, 0x200 LDS write, 0x002 VALU.
#define MOE_SG(mask, n) __builtin_amdgcn_sched_group_barrier(mask, n, 0)
#define MOE_PATTERN_LOAD()                                              \
  _Pragma("unroll") for (int i_ = 0; i_ < 8; ++i_) {                    \
    MOE_SG(0x008, 1); MOE_SG(0x020, 2); MOE_SG(0x100, 1);               \
  }                                                                     \
  _Pragma("unroll") for (int i_ = 0; i_ < 8; ++i_) MOE_SG(0x008, 1)
#define MOE_PATTERN_STORE()                                             \
  _Pragma("unroll") for (int i_ = 0; i_ < 8; ++i_) {                    \
    MOE_SG(0x008, 1); MOE_SG(0x100, 1); MOE_SG(0x002, 4); MOE_SG(0x200, 1); \
  }                                                                     \
  _Pragma("unroll") for (int i_ = 0; i_ < 8; ++i_) {                    \
    MOE_SG(0x008, 1); MOE_SG(0x002, 4); MOE_SG(0x200, 1);               \
  }
#define MOE_PATTERN_READ()                                              \
  _Pragma("unroll") for (int i_ = 0; i_ < 8; ++i_) {                    \
    MOE_SG(0x008, 1); MOE_SG(0x100, 1);                                 \
  }                                                                     \
  _Pragma("unroll") for (int i_ = 0; i_ < 8; ++i_) MOE_SG(0x008, 1)

#define MOE_STEP(L, S, st)                                              \
  do {                                                                  \
    MOE_GLOAD(L, min(kt + 2, nk - 1) * kBK);                            \
    MOE_LOADF(1, st, 1);                                                \
    MOE_MMA(0);                                                         \
    MOE_PATTERN_LOAD();                                                 \
    MOE_FENCE();                                                        \
    MOE_LOADF(0, st, 2);                                                \
    MOE_LSTORE(S, (st) ^ 1);                                            \
    MOE_MMA(1);                                                         \
    MOE_PATTERN_STORE();                                                \
    MOE_FENCE();                                                        \
    MOE_LOADF(1, st, 3);                                                \
    MOE_MMA(0);                                                         \
    MOE_PATTERN_READ();                                                 \
    MOE_FENCE();                                                        \
    __syncthreads();                                                    \
    MOE_FENCE();                                                        \
    MOE_LOADF(0, (st) ^ 1, 0);                                          \
    MOE_MMA(1);                                                         \
    MOE_PATTERN_READ();                                                 \
    MOE_FENCE();                                                        \
  } while (0)

  const int nk = K / kBK;
  MOE_GLOAD(x, 0);
  MOE_LSTORE(x, 0);
  MOE_GLOAD(y, min(1, nk - 1) * kBK);
  __syncthreads();
  MOE_LOADF(0, 0, 0);
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    MOE_STEP(x, y, 0);      // step kt   (even): stage 0, loads kt+2 -> x, stores y (kt+1)
    ++kt;
    MOE_STEP(y, x, 1);      // step kt+1 (odd) : stage 1, loads kt+3 -> y, stores x (kt+2)
    --kt;
  }
  if (kt < nk) MOE_STEP(x, y, 0);
#undef MOE_LOADF
#undef MOE_MMA
#undef MOE_FENCE
#undef MOE_SG
#undef MOE_PATTERN_LOAD
#undef MOE_PATTERN_STORE
#undef MOE_PATTERN_READ
#undef MOE_GLOAD
#undef MOE_LSTORE
#undef MOE_STEP

  // ---- epilogue
  if (UP) {
    uint16_t* act = static_cast<uint16_t*>(out);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = r0 + wm * 128 + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
        if (row < rend) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const float h1 = acc[i][j][r], h3 = acc[i][j + 2][r];
            const float gv = h1 * __builtin_amdgcn_rcpf(1.f + __expf(-h1)) * h3;
            act[(size_t)row * Nout + n0 + wn * 64 + 32 * j + l32] = f32_to_bf16(gv);
          }
        }
      }
  } else {
    float* y = static_cast<float*>(out);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = r0 + wm * 128 + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
        if (row < rend) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            y[(size_t)row * Nout + n0 + wn * 128 + 32 * j + l32] = acc[i][j][r];
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
                       n_tiles, max_rows, act);
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
                       d, n_tiles, max_rows, static_cast<void*>(y_perm));
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
