// Backward pass of the layer: gradients of L = <dy, y> + aux_coef * aux.
//
// The aux loss exists for training (cf-1.com/news/5914943 §2.3,
// hotelren.com/news/5904824 §3.2); every expert keeps gradients of its own
// (2kiu.com/news/2885792 §2.2) and only the selected experts receive any
// (2kiu.com/news/2885792 §5.1).  The weight gradients keep the weights'
// layout, one tensor per matrix sliced by expert (2kiu.com/news/2885792 §5.4):
// [N, d, f] for W1 and W3, [N, f, d] for W2, in fp32.
// The top-k choice, the capacity cut and the counts are piecewise constant:
// gradients reach the router through the softmax over the k selected logits
// and through the mean router probability in the aux loss.
//
// Steps (r = row of slot (t, j) in the expert-contiguous order, w = its gate
// weight, x = hidden[t], h1 = x W1_e, h3 = x W3_e, a = silu(h1) * h3):
//   combine  : g[r] = w * dy[t];  dgate[t, j] = <dy[t], y_perm[r]>
//   da       : da[r] = g[r] W2_e^T                              (grouped, NT)
//   swiglu   : recompute h1, h3; dh1 = da * h3 * silu'(h1), dh3 = da * silu(h1),
//              a = silu(h1) * h3                                 (grouped, NN)
//              (with h1, h3 saved by the forward: in the da GEMM's epilogue, and a
//              is the forward's own activation when the caller passes it)
//   dx       : dx[r] = dh1[r] W1_e^T + dh3[r] W3_e^T              (grouped, NT, K = 2f;
//              a sparse last round of deep tiles is split over k)
//   weights  : dW2_e = a_e^T g_e;  [dW1_e | dW3_e] = x_e^T [dh1_e | dh3_e]
//                                                   (per expert, k = the expert's rows)
//   router   : dlogit = softmax-over-k Jacobian of dgate + aux_coef * d aux / d logits;
//              dhidden[t] = sum_j dx[slot (t, j)] + dlogit[t] W_router^T;
//              dW_router = hidden^T dlogit;  dbias = sum_t dlogit[t]
//
// bf16 GEMMs run on one MFMA tile kernel with the forward's structure (256 x
// 256 tiles, 8 waves of 128 x 64 on 16x16x32 bf16 MFMAs, two 64 KB LDS stages
// filled by direct buffer -> LDS loads issued by one wave per SIMD) and a
// template per step that sets how
// each operand is laid out in memory: k-contiguous operands (x, g, dh rows;
// W2 and W1/W3 read as their transposes) are staged row-major and read with
// ds_read_b128; m- or n-contiguous operands (W1/W3 in the recompute, every
// operand of the weight gradients, whose depth is the expert's token rows)
// are staged k-row-major and read with the transposing ds_read_b64_tr_b16.
// The weight gradients' depth ends at the expert's last row: the buffer
// resource stops there, so the loads past it return zeros.
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace moe {
namespace bwd {

// kDAS: the da GEMM with the SwiGLU backward in its epilogue, from the h1 / h3
// the forward saved (moe_expert_backward_saved): no recompute GEMM
enum Mode { kDA = 0, kDX = 1, kSwiGLU = 2, kWGrad = 3, kDAS = 4 };

constexpr int kBM = 256, kBN = 256, kBK = 64, kThreads = 512, kGroupM = 8;
// transposed operand tile: 16-element (32-byte) pad after every 4 k-rows of 128
constexpr int kTGroup = 4 * 128 + 8, kTSub = 16 * kTGroup, kRegion = 2 * kTSub;
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// One GEMM launch.  Row indices r are rows of the expert-contiguous order.
struct Args {
  const void* a;            // A operand base
  int lda;                  // its row stride (elements)
  const void* b0;           // B operand (DX: W1 for k < ksplit steps; SwiGLU: W1)
  const void* b1;           // DX: W3; SwiGLU: W3
  int ldb;
  long long b_estride;      // elements between experts' weight matrices (grouped-row steps)
  const int32_t* offsets;
  int n_exp, max_rows;
  int K;                    // depth of the grouped-row steps
  int M;                    // WGrad: rows of each expert's output
  int Nn;                   // output columns (SwiGLU: f)
  int n_tiles;              // output column tiles (set by the launcher)
  int ksplit;               // DX: 64-deep k-steps read from b0 before b1
  float* out0;              // fp32 output (DA: da, DX: dx, WGrad: columns < nsplit)
  float* out1;              // WGrad: columns >= nsplit
  int ldo, nsplit;
  long long o_estride;      // WGrad: elements between experts' outputs
  const float* da;          // SwiGLU: da [rows, f] (input)
  const void* h13;          // DAS: [h1 | h3] [rows, 2f] saved by the forward (input)
  void* dh;                 // SwiGLU: [dh1 | dh3] [rows, 2f] (output)
  void* act;                // SwiGLU: a [rows, f] (output)
  int f;
  // DX: the last round's tiles split over k (partial tiles and one ticket per
  // compute unit in the workspace); null tickets: no split
  float* part;
  int32_t* tickets;
  int num_cus;
  int dp_grid;              // blocks [0, dp_grid) compute whole tiles
};

__device__ __forceinline__ bool dp_logical(int total, int& logical) {
  const int per = (total + 7) >> 3;
  const int b = blockIdx.x;
  const int local = b >> 3;
  if (local >= per) return false;
  logical = (b & 7) * per + local;
  return logical < total;
}

__device__ __forceinline__ void tile_of_logical(int logical, int m_tiles, int n_tiles, int& mt,
                                                int& nt) {
  const int span = kGroupM * n_tiles;
  const int grp = logical / span;
  const int first = grp * kGroupM;
  const int gm = (m_tiles - first) < kGroupM ? (m_tiles - first) : kGroupM;
  const int in = logical - grp * span;
  mt = first + in % gm;
  nt = in / gm;
}

__device__ __forceinline__ uint4 frag_tr(const uint16_t* p) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p + kTGroup));
  const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
  return make_uint4(l2.x, l2.y, h2.x, h2.y);
}

// Fragments of the 16x16x32 MFMA (lane l: row / column l % 16, k values
// 8 (l / 16) .. +7 of a 32-deep slice s).  A row blocks ib (16 rows each) and
// B column blocks jb (16 columns each); two base addresses per operand:
//   row-major A:  ab[s] + 4096 (ib / 2) + 1024 (ib % 2)
//   transposed A: ab[(ib / 2) % 2] + kTSub (ib / 4) + 16 (ib % 2) + 8 kTGroup s
//   row-major B:  bb[s] + 1024 jb
//   transposed B: bb[jb / 2] + 16 (jb % 2) + 8 kTGroup s
template <bool AT>
__device__ __forceinline__ uint4 rd_a(const uint16_t* __restrict__ st, const int (&ab)[2], int s, int ib) {
  if (AT) return frag_tr(st + ab[(ib >> 1) & 1] + kTSub * (ib >> 2) + 16 * (ib & 1) + 8 * kTGroup * s);
  return *reinterpret_cast<const uint4*>(st + ab[s] + 4096 * (ib >> 1) + 1024 * (ib & 1));
}
template <bool BT>
__device__ __forceinline__ uint4 rd_b(const uint16_t* __restrict__ st, const int (&bb)[2], int s, int jb) {
  const uint16_t* bs = st + kRegion;
  if (BT) return frag_tr(bs + bb[jb >> 1] + 16 * (jb & 1) + 8 * kTGroup * s);
  return *reinterpret_cast<const uint4*>(bs + bb[s] + 1024 * jb);
}

// The MFMAs of one slice for the NB row blocks that hold rows, each fragment
// register refilled with slice ns of stage nst right after its last use (A
// row block by row block, B during the last row block).
template <int NB, bool AT, bool BT>
__device__ __forceinline__ void slice_mma(uint4 (&fa)[8], uint4 (&fb)[4], f32x4 (&acc)[8][4],
                                          const uint16_t* __restrict__ nst, const int (&ab)[2],
                                          const int (&bb)[2], int ns) {
#pragma unroll
  for (int ib = 0; ib < NB; ++ib) {
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      acc[ib][jb] = mfma16(fa[ib], fb[jb], acc[ib][jb]);
      if (ib == NB - 1) fb[jb] = rd_b<BT>(nst, bb, ns, jb);
    }
    fa[ib] = rd_a<AT>(nst, ab, ns, ib);
  }
}

// Per-lane state of the direct loads issued by one loading wave: instruction i
// loads at  v[i % 2] + u + i * step + k-step offset  (the two per-lane variants
// are the swizzles of even and odd 8-row groups of a row-major operand and are
// equal for a transposed one).
struct Loader {
  __amdgpu_buffer_rsrc_t a_rs, b_rs0, b_rs1;
  uint32_t a_v0, a_v1, b_v0, b_v1;
  uint32_t a_u, a_step, b_u, b_step;
  uint32_t a_kstride, b_kstride;
  int ksplit;
  int kbase;                  // first k-step of this block's range
  int w;                      // loading wave 0..3
};

// LDS destination of load instruction ins = 8 w + i of an operand region:
// row-major 1 KB per instruction; transposed 4 k-rows of sub-tile ins / 16,
// each group of 4 k-rows followed by 16 bytes of padding.
template <bool TR>
__device__ __forceinline__ int ldst(int w, int i) {
  return TR ? kTSub * (w >> 1) + kTGroup * (8 * (w & 1) + i) : (8 * w + i) * 512;
}

template <bool AT, bool BT>
__device__ __forceinline__ void issue(uint16_t* __restrict__ dst, const Loader& L, int kstep) {
  kstep += L.kbase;
  const uint32_t ka = (uint32_t)kstep * L.a_kstride;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(L.a_rs, (lds_void*)(dst + ldst<AT>(L.w, i)), 16,
                                             ((i & 1) ? L.a_v1 : L.a_v0) + (L.a_u + i * L.a_step + ka),
                                             0, 0, 0);
  const bool hi = kstep >= L.ksplit;
  const __amdgpu_buffer_rsrc_t b_rs = hi ? L.b_rs1 : L.b_rs0;
  const uint32_t kb = (uint32_t)(hi ? kstep - L.ksplit : kstep) * L.b_kstride;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rs, (lds_void*)(dst + kRegion + ldst<BT>(L.w, i)),
                                             16, ((i & 1) ? L.b_v1 : L.b_v0) + (L.b_u + i * L.b_step + kb),
                                             0, 0, 0);
}

#define MOE_BWD_WAIT_BARRIER() asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory")

// One 64-deep k-step (the forward GEMM's schedule: two 32-deep slices): fa/fb
// hold slice 0 of `cur` on entry; after the barrier that follows the last
// read of `cur`, the loading waves refill `cur` two steps ahead, interleaved
// with slice 1's MFMAs, while slice 0 of `nxt` is read.
template <int NB, bool DMA, bool AT, bool BT>
__device__ __forceinline__ void kstep_body(const uint16_t* __restrict__ cur,
                                           uint16_t* __restrict__ dst,
                                           const uint16_t* __restrict__ nxt, const Loader& L,
                                           int kstep, const int (&ab)[2], const int (&bb)[2],
                                           f32x4 (&acc)[8][4], uint4 (&fa)[8], uint4 (&fb)[4]) {
  if (NB > 0) slice_mma<NB, AT, BT>(fa, fb, acc, cur, ab, bb, 1);
  MOE_BWD_WAIT_BARRIER();
  if (DMA && NB == 8) {
    issue<AT, BT>(dst, L, kstep);
    slice_mma<NB, AT, BT>(fa, fb, acc, nxt, ab, bb, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  } else {
    if (DMA) issue<AT, BT>(dst, L, kstep);
    __builtin_amdgcn_sched_barrier(0);
    if (NB > 0) slice_mma<NB, AT, BT>(fa, fb, acc, nxt, ab, bb, 0);
  }
}

__device__ __forceinline__ int clamp_off(const int32_t* offsets, int e, int max_rows, int lo) {
  return min(max(offsets[e], lo), max_rows);
}

// Split of the last round of tiles over k (dx only: 1088 tiles of 448 k-steps
// at the Mixtral counts leave a last round of 64 tiles on 256 CUs): when the
// last round would leave at least half of the CUs idle, each of its r tiles is
// cut into up to 4 k-ranges run by separate blocks, and the last block of a
// tile to take its ticket sums the partial tiles in range order (the forward
// down projection's scheme; results do not depend on which block finishes
// last).  Only tiles of at least 128 k-steps are split.  Returns the number of
// tiles computed whole.
constexpr int kMaxSegs = 4, kMinSplitSteps = 128;
__device__ __forceinline__ int split_plan(int total, int nk, int num_cus, int& segs) {
  segs = 1;
  if (num_cus <= 0 || nk < kMinSplitSteps) return total;
  const int r = total % num_cus;
  if (r == 0 || 2 * r > num_cus) return total;
  int sg = num_cus / r;
  sg = sg < kMaxSegs ? sg : kMaxSegs;
  sg = sg < nk / 2 ? sg : nk / 2;
  if (sg < 2) return total;
  segs = sg;
  return total - r;
}

// LDS layout of one stage: A region at element 0, B region at kRegion.
//   row-major operand  [256 rows][64 k]: chunk c of row r at position c ^ ((r >> 1) & 7)
//   transposed operand 2 x [64 k][128 cols]: chunk c of k-row kr at c ^ (4 (kr & 3)),
//     every 4 k-rows followed by 16 bytes of padding (a 32-lane half of a
//     transposing read covers k rows r .. r+3 and r+8 .. r+11, which share the
//     swizzle; the padding moves the second group to other banks)
template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void bwd_gemm_bf16_kernel(Args p) {
  constexpr bool AT = MODE == kWGrad;                       // A m-contiguous
  constexpr bool BT = MODE == kSwiGLU || MODE == kWGrad;    // B n-contiguous
  constexpr bool GK = MODE == kWGrad;                       // depth = the expert's rows
  __shared__ __align__(1024) uint16_t S0[2 * kRegion], S1[2 * kRegion];
  __shared__ int s_last;

  int e, r0, rend, mt, nt, m0 = 0, kl, kb = 0, slot = -1, segs = 1;
  if (GK) {
    const int m_tiles = p.M / kBM;
    const int tpe = m_tiles * p.n_tiles;
    int logical;
    if (!dp_logical(tpe * p.n_exp, logical)) return;
    e = logical / tpe;
    tile_of_logical(logical - e * tpe, m_tiles, p.n_tiles, mt, nt);
    r0 = clamp_off(p.offsets, e, p.max_rows, 0);
    rend = min(max(p.offsets[e + 1], r0), p.max_rows);
    m0 = mt * kBM;
    kl = (rend - r0 + kBK - 1) / kBK;
  } else {
    const int m_tiles = count_tiles(p.offsets, p.n_exp, kBM, p.max_rows);
    const int total = m_tiles * p.n_tiles;
    const int nk = p.K / kBK;
    const int n_dp = (MODE == kDX && p.tickets) ? split_plan(total, nk, p.num_cus, segs) : total;
    // blocks [0, dp_grid) compute whole tiles; the rest compute k-ranges of the
    // last tiles (block j: tile n_dp + j / segs, range j % segs)
    int logical;
    kl = nk;
    if (MODE != kDX || (int)blockIdx.x < p.dp_grid) {
      if (!dp_logical(n_dp, logical)) return;
    } else {
      const int j = blockIdx.x - p.dp_grid;
      if (j >= (total - n_dp) * segs) return;
      logical = n_dp + j / segs;
      const int seg = j % segs;
      kb = seg * nk / segs;
      kl = (seg + 1) * nk / segs - kb;
      slot = j;
    }
    tile_of_logical(logical, m_tiles, p.n_tiles, mt, nt);
    if (!find_tile(p.offsets, p.n_exp, mt, kBM, p.max_rows, e, r0, rend)) return;
  }
  kb = __builtin_amdgcn_readfirstlane(kb);
  slot = __builtin_amdgcn_readfirstlane(slot);
  e = __builtin_amdgcn_readfirstlane(e);
  r0 = __builtin_amdgcn_readfirstlane(r0);
  rend = __builtin_amdgcn_readfirstlane(rend);
  nt = __builtin_amdgcn_readfirstlane(nt);
  m0 = __builtin_amdgcn_readfirstlane(m0);
  kl = __builtin_amdgcn_readfirstlane(kl);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sm = w & 3, pw = w >> 2;
  const int wm = sm & 1, wn = sm >> 1;
  const int n0 = MODE == kSwiGLU ? nt * (kBN / 2) : nt * kBN;
  const int rows = rend - r0;
  const int tile_rows = min(rows, kBM);

  // ---- load set-up (only waves 0..3 issue loads)
  Loader L;
  L.w = w & 3;
  L.ksplit = MODE == kDX ? p.ksplit : 0x7FFFFFFF;
  L.kbase = kb;
  const uint16_t* A = static_cast<const uint16_t*>(p.a) + (size_t)r0 * p.lda;
  // rows past the tile's end (and, for the weight gradients, k rows past the
  // expert's last row) lie outside the resource's range and load as zeros
  L.a_rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(A), 0,
                                             (GK ? rows : tile_rows) * p.lda * 2, kRsrcWord3);
  if (GK) {
    const uint16_t* B = static_cast<const uint16_t*>(p.b0) + (size_t)r0 * p.ldb;
    L.b_rs0 = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(B), 0, rows * p.ldb * 2,
                                                kRsrcWord3);
    L.b_rs1 = L.b_rs0;
  } else {
    const size_t wexp = (size_t)e * p.b_estride;
    const int wbytes = (int)(p.b_estride * 2);
    L.b_rs0 = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(static_cast<const uint16_t*>(p.b0) + wexp), 0, wbytes, kRsrcWord3);
    L.b_rs1 = MODE == kSwiGLU || MODE == kDX
                  ? __builtin_amdgcn_make_buffer_rsrc(
                        const_cast<uint16_t*>(static_cast<const uint16_t*>(p.b1) + wexp), 0,
                        wbytes, kRsrcWord3)
                  : L.b_rs0;
  }
  L.a_kstride = AT ? (uint32_t)(kBK * p.lda * 2) : (uint32_t)(kBK * 2);
  L.b_kstride = BT ? (uint32_t)(kBK * p.ldb * 2) : (uint32_t)(kBK * 2);
  {
    // instruction ins = 8 w + i.  Row-major operand: rows 8 ins + lane / 8, chunk
    // (lane % 8) ^ ((row / 2) % 8) = (lane % 8) ^ (4 (i % 2) + lane / 16).
    // Transposed operand: sub-tile ins / 16 (= w / 2), k rows 4 (ins % 16) + lane / 16,
    // chunk (lane % 16) ^ (4 (lane / 16)).
    const int wl = L.w;
    const int cbt = (lane & 15) ^ (4 * (lane >> 4));
    if (AT) {
      L.a_v0 = L.a_v1 = (uint32_t)(((lane >> 4) * p.lda + 8 * cbt) * 2);
      L.a_u = (uint32_t)((32 * (wl & 1) * p.lda + m0 + 128 * (wl >> 1)) * 2);
      L.a_step = (uint32_t)(8 * p.lda);
    } else {
      const int rl = lane >> 3;
      L.a_v0 = (uint32_t)((rl * p.lda + 8 * ((lane & 7) ^ (lane >> 4))) * 2);
      L.a_v1 = (uint32_t)((rl * p.lda + 8 * ((lane & 7) ^ (4 + (lane >> 4)))) * 2);
      L.a_u = (uint32_t)(16 * p.lda * 8 * wl);
      L.a_step = (uint32_t)(16 * p.lda);
    }
    if (BT) {
      L.b_v0 = L.b_v1 = (uint32_t)(((lane >> 4) * p.ldb + 8 * cbt) * 2);
      const int colbase = MODE == kSwiGLU ? n0 : n0 + 128 * (wl >> 1);
      L.b_u = (uint32_t)((32 * (wl & 1) * p.ldb + colbase) * 2);
      L.b_step = (uint32_t)(8 * p.ldb);
    } else {
      const int rl = lane >> 3;
      L.b_v0 = (uint32_t)((rl * p.ldb + 8 * ((lane & 7) ^ (lane >> 4))) * 2);
      L.b_v1 = (uint32_t)((rl * p.ldb + 8 * ((lane & 7) ^ (4 + (lane >> 4)))) * 2);
      L.b_u = (uint32_t)((n0 + 64 * wl) * p.ldb * 2);
      L.b_step = (uint32_t)(16 * p.ldb);
    }
  }
  if (MODE == kSwiGLU && (L.w >> 1)) L.b_rs0 = L.b_rs1;     // sub-tile 1 holds the W3 columns

  // ---- fragment base addresses (element offsets inside a stage)
  int ab[2], bb[2];
  {
    const int gq = lane >> 4, i16 = lane & 15;
    const int kr = 8 * gq + (i16 >> 2);                     // transposed reads: k row of the lane
    if (AT) {
      // row block ib: tile rows 64 (ib / 2) + 32 wm + 16 (ib % 2); base per (ib / 2) % 2
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const int col = 64 * hb + 32 * wm + 4 * (i16 & 3);
        ab[hb] = (kr >> 2) * kTGroup + (kr & 3) * 128 + 8 * ((col >> 3) ^ (4 * (kr & 3))) + (col & 7);
      }
    } else {
      const int row = 32 * wm + i16;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) ab[s2] = row * 64 + 8 * ((4 * s2 + gq) ^ ((row >> 1) & 7));
    }
    if (BT) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int q = MODE == kSwiGLU ? j : wn;
        const int cb = MODE == kSwiGLU ? (wn * 64 + 32 * pw) : (64 * pw + 32 * j);
        const int col = cb + 4 * (i16 & 3);
        bb[j] = q * kTSub + (kr >> 2) * kTGroup + (kr & 3) * 128 + 8 * ((col >> 3) ^ (4 * (kr & 3))) +
                (col & 7);
      }
    } else {
      const int row = wn * 128 + 64 * pw + i16;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) bb[s2] = row * 64 + 8 * ((4 * s2 + gq) ^ ((row >> 1) & 7));
    }
  }

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.f;

  const int nv = GK ? 4 : __builtin_amdgcn_readfirstlane(min(4, max(0, (tile_rows - 32 * wm + 63) / 64)));
#define MOE_BWD_KLOOP(NV, D)                                                               \
  do {                                                                                     \
    uint4 fa[8], fb[4];                                                                    \
    _Pragma("unroll") for (int ib = 0; ib < 2 * NV; ++ib) fa[ib] = rd_a<AT>(S0, ab, 0, ib); \
    _Pragma("unroll") for (int jb = 0; jb < 4; ++jb) fb[jb] = rd_b<BT>(S0, bb, 0, jb);     \
    int kt = 0;                                                                            \
    for (; kt + 2 <= kl; kt += 2) {                                                        \
      kstep_body<2 * NV, D, AT, BT>(S0, S0, S1, L, min(kt + 2, kl - 1), ab, bb, acc, fa, fb); \
      kstep_body<2 * NV, D, AT, BT>(S1, S1, S0, L, min(kt + 3, kl - 1), ab, bb, acc, fa, fb); \
    }                                                                                      \
    if (kt < kl)                                                                           \
      kstep_body<2 * NV, D, AT, BT>(S0, S0, S1, L, min(kt + 2, kl - 1), ab, bb, acc, fa, fb); \
  } while (0)
  if (kl > 0) {
    if (pw == 0) {
      issue<AT, BT>(S0, L, 0);
      issue<AT, BT>(S1, L, min(1, kl - 1));
      asm volatile("s_waitcnt vmcnt(16) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      switch (nv) {
        case 4: MOE_BWD_KLOOP(4, true); break;
        case 3: MOE_BWD_KLOOP(3, true); break;
        case 2: MOE_BWD_KLOOP(2, true); break;
        case 1: MOE_BWD_KLOOP(1, true); break;
        default: MOE_BWD_KLOOP(0, true); break;
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);        // vmcnt(0): no LDS write in flight at exit
    } else {
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      switch (nv) {
        case 4: MOE_BWD_KLOOP(4, false); break;
        case 3: MOE_BWD_KLOOP(3, false); break;
        case 2: MOE_BWD_KLOOP(2, false); break;
        case 1: MOE_BWD_KLOOP(1, false); break;
        default: MOE_BWD_KLOOP(0, false); break;
      }
    }
  }
#undef MOE_BWD_KLOOP

  // ---- dx k-range blocks: store the partial tile; the last of a tile's
  // blocks to take its ticket sums all of the tile's partials in range order
  // and goes on to the normal epilogue
  if (MODE == kDX && slot >= 0) {
    const __amdgpu_buffer_rsrc_t mine = __builtin_amdgcn_make_buffer_rsrc(
        p.part + (size_t)slot * (kBM * kBN), 0, kBM * kBN * 4, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = acc[i][j][r];
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), mine, tid * 4,
                                                ((i * 4 + j) * 4 + r) * kThreads * 4, 0);
        }
    // every wave's stores are done before the barrier; one wave then makes the
    // block's tile visible device-wide and takes the ticket
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int tile_sk = slot / segs;
    if (tid == 0) {
      __threadfence();
      const int last = atomicAdd(&p.tickets[tile_sk], 1) == segs - 1;
      if (last) __threadfence();       // acquire the other blocks' partial tiles
      s_last = last;
    }
    __syncthreads();
    if (!s_last) return;
    const __amdgpu_buffer_rsrc_t all = __builtin_amdgcn_make_buffer_rsrc(
        p.part + (size_t)tile_sk * segs * (kBM * kBN), 0, segs * kBM * kBN * 4, kRsrcWord3);
    for (int q = 0; q < segs; ++q) {
      const int qo = q * kBM * kBN * 4;
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float v = __builtin_bit_cast(
                float, __builtin_amdgcn_raw_buffer_load_b32(all, tid * 4,
                                                            qo + ((i * 4 + j) * 4 + r) * kThreads * 4, 0));
            acc[i][j][r] = q == 0 ? v : acc[i][j][r] + v;
          }
    }
  }

  // ---- epilogues.  acc[ib][jb][r]: tile row 64 (ib / 2) + 32 wm + 16 (ib % 2) + 4 (lane / 16) + r,
  // column 16 jb + lane % 16 of the wave's 64 columns (SwiGLU: jb < 2 W1, jb >= 2 the same W3 columns)
  const int l16 = lane & 15, g4 = 4 * (lane >> 4);
  if (MODE == kSwiGLU) {
    // Stage the tile's da block (256 rows x 128 fp32 columns, 128 KB) in the
    // two LDS stages with direct loads from every wave, so that the epilogue
    // does not wait on dependent global loads: after every fragment read and
    // every refill is done, wave w loads rows 32 w .. 32 w + 31 (two 512-byte
    // rows per 1 KB instruction; rows past the tile read zeros).
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    {
      const __amdgpu_buffer_rsrc_t da_rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(p.da + (size_t)r0 * p.f + n0), 0, tile_rows * p.f * 4, kRsrcWord3);
      const uint32_t vo = (uint32_t)(((32 * w + (lane >> 5)) * p.f + 4 * (lane & 31)) * 4);
      uint16_t* dst = (w < 4 ? S0 : S1) + (w & 3) * 8192;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(da_rs, (lds_void*)(dst + i * 512), 16, vo,
                                                 (uint32_t)(2 * i * p.f * 4), 0, 0);
    }
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    const float* da0 = reinterpret_cast<const float*>(S0);
    const float* da1 = reinterpret_cast<const float*>(S1);
    uint16_t* dh = static_cast<uint16_t*>(p.dh);
    uint16_t* act = static_cast<uint16_t*>(p.act);
    const int f = p.f;
#pragma unroll
    for (int ib = 0; ib < 8; ++ib)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tr = 64 * (ib >> 1) + 32 * wm + 16 * (ib & 1) + g4 + r;
        const int row = r0 + tr;
        if (row < rend) {
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int cl = wn * 64 + 32 * pw + 16 * jj + l16;
            const int col = n0 + cl;
            const float h1 = acc[ib][jj][r], h3 = acc[ib][2 + jj][r];
            const float g = ib < 4 ? da0[tr * 128 + cl] : da1[(tr - 128) * 128 + cl];
            const float s = __builtin_amdgcn_rcpf(1.f + __expf(-h1));
            const float sl = h1 * s;
            dh[(size_t)row * 2 * f + col] = f32_to_bf16(g * h3 * (s + sl * (1.f - s)));
            dh[(size_t)row * 2 * f + f + col] = f32_to_bf16(g * sl);
            act[(size_t)row * f + col] = f32_to_bf16(sl * h3);
          }
        }
      }
  } else if (MODE == kDAS) {
    // acc = da for tile rows x f-columns n0 .. n0 + 255.  Four passes of 64 tile rows
    // (row blocks ib = 2 pass, 2 pass + 1):
    //  1. the rows' saved [h1 256 | h3 256] (bf16, 1 KB) come into LDS by direct loads
    //     from every wave (8 rows each, one row per 1 KB instruction: lanes 0..31 read
    //     the h1 piece, 32..63 the h3 piece; rows past the tile read zeros);
    //  2. each lane turns its h1, h3 and da into dh1, dh3 (written over h1, h3) and,
    //     unless the caller passed the forward's activations, a (into S1, 512-byte
    //     rows plus 16 bytes of padding);
    //  3. the block writes the rows' dh1, dh3 (and a) pieces (512 bytes each) to global
    //     memory with 16-byte stores (2-byte stores from the accumulators' lanes cost a
    //     quarter of this GEMM).
    // Without a, the passes alternate between the two stages and the next pass's
    // rows load while the current pass computes and stores; with a, S1 holds the
    // a rows and every pass loads into S0 after the previous pass's stores.
    constexpr int kActE = 264;
    const int f = p.f;
    const bool want_act = p.act != nullptr;      // block-uniform
    const __amdgpu_buffer_rsrc_t h_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(static_cast<const uint16_t*>(p.h13) + (size_t)r0 * 2 * f), 0,
        tile_rows * 2 * f * 2, kRsrcWord3);
    const uint32_t hv = (uint32_t)((((lane >> 5) ? f : 0) + n0 + 8 * (lane & 31)) * 2);
    // stores past the tile's last row fall outside the range and are dropped, so
    // every wave issues the same number of stores per pass
    const __amdgpu_buffer_rsrc_t dh_rs = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<uint16_t*>(p.dh) + (size_t)r0 * 2 * f, 0, tile_rows * 2 * f * 2, kRsrcWord3);
    uint16_t* act = static_cast<uint16_t*>(p.act);
    auto load_pass = [&](uint16_t* buf, int pass) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            h_rs, (lds_void*)(buf + (8 * w + i) * 512), 16, hv,
            (uint32_t)((64 * pass + 8 * w + i) * 2 * f * 2), 0, 0);
    };
    // every h1 / h3 of the lane is read before the first dh is written over them,
    // so the reads issue back to back instead of each waiting out the LDS latency
    auto compute_pass = [&](uint16_t* hbuf, int pass) {
      uint16_t hv[2][4][4][2];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int jb = 0; jb < 4; ++jb) {
            const int lr = 32 * wm + 16 * b + g4 + r;
            const int cl = wn * 128 + 64 * pw + 16 * jb + l16;
            hv[b][r][jb][0] = hbuf[lr * 512 + cl];
            hv[b][r][jb][1] = hbuf[lr * 512 + 256 + cl];
          }
#pragma unroll
      for (int ib = 2 * pass; ib < 2 * pass + 2; ++ib)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int lr = 32 * wm + 16 * (ib & 1) + g4 + r;        // row within the pass
          uint16_t* hrow = hbuf + lr * 512;
          uint16_t* arow = S1 + lr * kActE;
#pragma unroll
          for (int jb = 0; jb < 4; ++jb) {
            const int cl = wn * 128 + 64 * pw + 16 * jb + l16;
            const float h1 = bf16_to_f32(hv[ib & 1][r][jb][0]);
            const float h3 = bf16_to_f32(hv[ib & 1][r][jb][1]);
            const float g = acc[ib][jb][r];
            const float sg = __builtin_amdgcn_rcpf(1.f + __expf(-h1));
            const float sl = h1 * sg;
            hrow[cl] = f32_to_bf16(g * h3 * (sg + sl * (1.f - sg)));
            hrow[256 + cl] = f32_to_bf16(g * sl);
            if (want_act) arow[cl] = f32_to_bf16(sl * h3);
          }
        }
    };
    // wave w: rows 8 w .. 8 w + 7 of the pass, 24 (row, piece) pairs (16 without
    // a), two per instruction (32 lanes x 16 bytes each)
    auto store_pieces = [&](const uint16_t* hbuf, int pass, auto pieces_c) {
      constexpr int pieces = decltype(pieces_c)::value;
      u32x4 pv[4 * pieces];      // every piece is read before the first store is issued
#pragma unroll
      for (int i = 0; i < 4 * pieces; ++i) {
        const int idx = 2 * i + (lane >> 5);
        const int prow = 8 * w + idx / pieces, seg = idx % pieces;
        const int c8 = 8 * (lane & 31);
        const uint16_t* src =
            seg == 2 ? S1 + prow * kActE + c8 : hbuf + prow * 512 + 256 * seg + c8;
        pv[i] = *reinterpret_cast<const u32x4*>(src);
      }
#pragma unroll
      for (int i = 0; i < 4 * pieces; ++i) {
        const int idx = 2 * i + (lane >> 5);
        const int prow = 8 * w + idx / pieces, seg = idx % pieces;
        const int trow = 64 * pass + prow;
        const int c8 = 8 * (lane & 31);
        const u32x4 v = pv[i];
        if (seg == 2) {
          if (r0 + trow < rend)
            *reinterpret_cast<u32x4*>(act + (size_t)(r0 + trow) * f + n0 + c8) = v;
        } else {
          __builtin_amdgcn_raw_buffer_store_b128(
              v, dh_rs, (uint32_t)(((size_t)trow * 2 * f + (seg == 1 ? f : 0) + n0 + c8) * 2), 0, 0);
        }
      }
    };
    if (want_act) {
#pragma unroll
      for (int pass = 0; pass < 4; ++pass) {
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        load_pass(S0, pass);
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        compute_pass(S0, pass);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        store_pieces(S0, pass, std::integral_constant<int, 3>{});
      }
    } else {
      // vector-memory operations of one wave, in issue order: L0 L1 | st0 L2 | st1 L3 |
      // st2 | st3 (Lp: 8 loads of pass p, stp: 8 stores of pass p); each wait lets the
      // operations issued after the pass's loads stay in flight
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      load_pass(S0, 0);
      load_pass(S1, 1);
      asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
      compute_pass(S0, 0);
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      store_pieces(S0, 0, std::integral_constant<int, 2>{});
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      load_pass(S0, 2);
      asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
      compute_pass(S1, 1);
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      store_pieces(S1, 1, std::integral_constant<int, 2>{});
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      load_pass(S1, 3);
      asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
      compute_pass(S0, 2);
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      store_pieces(S0, 2, std::integral_constant<int, 2>{});
      asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
      compute_pass(S1, 3);
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      store_pieces(S1, 3, std::integral_constant<int, 2>{});
    }
  } else if (MODE == kWGrad) {
    const bool low = n0 < p.nsplit;
    float* o = (low ? p.out0 : p.out1) + (size_t)e * p.o_estride;
    const int cbase = (low ? n0 : n0 - p.nsplit) + wn * 128 + 64 * pw + l16;
#pragma unroll
    for (int ib = 0; ib < 8; ++ib)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + 64 * (ib >> 1) + 32 * wm + 16 * (ib & 1) + g4 + r;
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) o[(size_t)row * p.ldo + cbase + 16 * jb] = acc[ib][jb][r];
      }
  } else {
    const int cbase = n0 + wn * 128 + 64 * pw + l16;
#pragma unroll
    for (int ib = 0; ib < 8; ++ib)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = r0 + 64 * (ib >> 1) + 32 * wm + 16 * (ib & 1) + g4 + r;
        if (row < rend) {
#pragma unroll
          for (int jb = 0; jb < 4; ++jb) p.out0[(size_t)row * p.ldo + cbase + 16 * jb] = acc[ib][jb][r];
        }
      }
  }
}

// ---------------------------------------------------------------- fp32 (VALU)
// The same four steps on 64 x 64 tiles, one k element at a time from LDS.
constexpr int kFB = 64, kFK = 16;

template <int MODE>
__global__ __launch_bounds__(256) void bwd_gemm_f32_kernel(Args p) {
  constexpr bool GK = MODE == kWGrad;
  __shared__ float As[kFK][kFB + 1];
  __shared__ float B0[kFK][kFB + 1];
  __shared__ float B1[kFK][kFB + 1];
  const float* a = static_cast<const float*>(p.a);
  const float* b0 = static_cast<const float*>(p.b0);
  const float* b1 = static_cast<const float*>(p.b1);
  int e, r0, rend, m0 = 0, depth;
  const int nt = blockIdx.y;
  if (GK) {
    e = blockIdx.z;
    m0 = blockIdx.x * kFB;
    r0 = clamp_off(p.offsets, e, p.max_rows, 0);
    rend = min(max(p.offsets[e + 1], r0), p.max_rows);
    depth = (rend - r0 + kFK - 1) / kFK * kFK;
  } else {
    if (!find_tile(p.offsets, p.n_exp, blockIdx.x, kFB, p.max_rows, e, r0, rend)) return;
    depth = p.K;
  }
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int n0 = nt * kFB;
  const size_t wexp = (size_t)e * p.b_estride;
  float c0[4][4] = {}, c1[4][4] = {};
  for (int k0 = 0; k0 < depth; k0 += kFK) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int item = tid + 256 * q;          // 64 x 16 items
      const int mm = item >> 4, kk = item & 15;      // A: row mm, depth kk
      const int kr = item >> 6, nn = item & 63;      // B: depth kr, column nn
      const int kA = k0 + kk, kB = k0 + kr;
      float av, bv0, bv1 = 0.f;
      if (GK) {
        av = r0 + kA < rend ? a[(size_t)(r0 + kA) * p.lda + m0 + mm] : 0.f;
        bv0 = r0 + kB < rend ? b0[(size_t)(r0 + kB) * p.ldb + n0 + nn] : 0.f;
      } else {
        av = r0 + mm < rend ? a[(size_t)(r0 + mm) * p.lda + kA] : 0.f;
        if (MODE == kSwiGLU) {
          bv0 = b0[wexp + (size_t)kB * p.ldb + n0 + nn];
          bv1 = b1[wexp + (size_t)kB * p.ldb + n0 + nn];
        } else if (MODE == kDX) {
          const int kf = p.ksplit * kBK;             // = f
          bv0 = kB < kf ? b0[wexp + (size_t)(n0 + nn) * p.ldb + kB]
                        : b1[wexp + (size_t)(n0 + nn) * p.ldb + kB - kf];
        } else {
          bv0 = b0[wexp + (size_t)(n0 + nn) * p.ldb + kB];
        }
      }
      As[kk][mm] = av;
      B0[kr][nn] = bv0;
      B1[kr][nn] = bv1;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kFK; ++kk) {
      float av[4], bv[4], bw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bv[j] = B0[kk][tx * 4 + j];
        bw[j] = B1[kk][tx * 4 + j];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          c0[i][j] = fmaf(av[i], bv[j], c0[i][j]);
          if (MODE == kSwiGLU) c1[i][j] = fmaf(av[i], bw[j], c1[i][j]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int mloc = ty * 4 + i;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      if (GK) {
        const bool low = n0 < p.nsplit;
        float* o = (low ? p.out0 : p.out1) + (size_t)e * p.o_estride;
        o[(size_t)(m0 + mloc) * p.ldo + (low ? col : col - p.nsplit)] = c0[i][j];
        continue;
      }
      const int row = r0 + mloc;
      if (row >= rend) continue;
      if (MODE == kDAS) {
        const int f = p.f;
        const float* hs = static_cast<const float*>(p.h13);
        const float h1 = hs[(size_t)row * 2 * f + col], h3 = hs[(size_t)row * 2 * f + f + col];
        const float g = c0[i][j];
        const float s = 1.f / (1.f + expf(-h1));
        const float sl = h1 * s;
        float* dh = static_cast<float*>(p.dh);
        dh[(size_t)row * 2 * f + col] = g * h3 * (s + sl * (1.f - s));
        dh[(size_t)row * 2 * f + f + col] = g * sl;
        if (p.act) static_cast<float*>(p.act)[(size_t)row * f + col] = sl * h3;
      } else if (MODE == kSwiGLU) {
        const int f = p.f;
        const float h1 = c0[i][j], h3 = c1[i][j];
        const float g = p.da[(size_t)row * f + col];
        const float s = 1.f / (1.f + expf(-h1));
        const float sl = h1 * s;
        float* dh = static_cast<float*>(p.dh);
        dh[(size_t)row * 2 * f + col] = g * h3 * (s + sl * (1.f - s));
        dh[(size_t)row * 2 * f + f + col] = g * sl;
        static_cast<float*>(p.act)[(size_t)row * f + col] = sl * h3;
      } else {
        p.out0[(size_t)row * p.ldo + col] = c0[i][j];
      }
    }
  }
}

// ---------------------------------------------------------------- combine backward
// One wave per token: g[r] = w * dy[t] and dgate[t, j] = <dy[t], y_perm[r]>
// (a fixed butterfly sum), 0 for dropped slots.
template <bool BF16>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const void* __restrict__ dy,
                                                          const float* __restrict__ y_perm,
                                                          const int32_t* __restrict__ slot_row,
                                                          const float* __restrict__ topk_w, int T,
                                                          int d, int k, void* __restrict__ g,
                                                          float* __restrict__ dgate) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  for (int j = 0; j < k; ++j) {
    const int r = slot_row[(size_t)t * k + j];
    if (r < 0) {
      if (lane == 0) dgate[(size_t)t * k + j] = 0.f;
      continue;
    }
    const float w = topk_w[(size_t)t * k + j];
    float dot = 0.f;
    for (int c = 8 * lane; c < d; c += 512) {
      float v[8];
      if (BF16) {
        const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(dy) + (size_t)t * d + c);
        v[0] = bf16lo(u.x); v[1] = bf16hi(u.x); v[2] = bf16lo(u.y); v[3] = bf16hi(u.y);
        v[4] = bf16lo(u.z); v[5] = bf16hi(u.z); v[6] = bf16lo(u.w); v[7] = bf16hi(u.w);
      } else {
        const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(dy) + (size_t)t * d + c);
        const float4 x0 = src[0], x1 = src[1];
        v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w;
        v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
      }
      const float4* yp = reinterpret_cast<const float4*>(y_perm + (size_t)r * d + c);
      const float4 y0 = yp[0], y1 = yp[1];
      dot = fmaf(v[0], y0.x, dot); dot = fmaf(v[1], y0.y, dot);
      dot = fmaf(v[2], y0.z, dot); dot = fmaf(v[3], y0.w, dot);
      dot = fmaf(v[4], y1.x, dot); dot = fmaf(v[5], y1.y, dot);
      dot = fmaf(v[6], y1.z, dot); dot = fmaf(v[7], y1.w, dot);
      if (BF16) {
        const uint4 pk = make_uint4(pack_bf16x2(w * v[0], w * v[1]), pack_bf16x2(w * v[2], w * v[3]),
                                    pack_bf16x2(w * v[4], w * v[5]), pack_bf16x2(w * v[6], w * v[7]));
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(g) + (size_t)r * d + c) = pk;
      } else {
        float4* dst = reinterpret_cast<float4*>(static_cast<float*>(g) + (size_t)r * d + c);
        dst[0] = make_float4(w * v[0], w * v[1], w * v[2], w * v[3]);
        dst[1] = make_float4(w * v[4], w * v[5], w * v[6], w * v[7]);
      }
    }
    dot = wave_sum(dot);
    if (lane == 0) dgate[(size_t)t * k + j] = dot;
  }
}

// ---------------------------------------------------------------- router backward
// One thread per token: dlogit[t, :] =
//   aux_coef * (N / T) * p[t, e] * (f_e - sum_m p[t, m] f_m)        (p = softmax of all N)
//   + at each selected id i_j: w_j * (dgate_j - sum_m w_m dgate_m)   (softmax over k)
__global__ __launch_bounds__(256) void router_dlogit_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ topk_w, const int32_t* __restrict__ counts,
    const float* __restrict__ dgate, float aux_coef, int T, int N, int k, float* __restrict__ dlog) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  const float* L = logits + (size_t)t * N;
  float* D = dlog + (size_t)t * N;
  if (aux_coef != 0.f) {
    float m = L[0];
    for (int e = 1; e < N; ++e) m = fmaxf(m, L[e]);
    float z = 0.f, pf = 0.f;
    const float inv_tk = 1.f / ((float)T * (float)k);
    for (int e = 0; e < N; ++e) {
      const float x = expf(L[e] - m);
      z += x;
      pf += x * ((float)counts[e] * inv_tk);
    }
    const float rz = 1.f / z;
    pf *= rz;
    const float scale = aux_coef * (float)N / (float)T;
    for (int e = 0; e < N; ++e) {
      const float pe = expf(L[e] - m) * rz;
      D[e] = scale * pe * ((float)counts[e] * inv_tk - pf);
    }
  } else {
    for (int e = 0; e < N; ++e) D[e] = 0.f;
  }
  float inner = 0.f;
  for (int j = 0; j < k; ++j) inner = fmaf(topk_w[(size_t)t * k + j], dgate[(size_t)t * k + j], inner);
  for (int j = 0; j < k; ++j) {
    const int e = topk_idx[(size_t)t * k + j];
    const float wj = topk_w[(size_t)t * k + j];
    D[e] += wj * (dgate[(size_t)t * k + j] - inner);
  }
}

// dhidden for 8 tokens x 1024 columns per block (4 adjacent columns per
// thread, 16-byte loads and stores): the router term dlogit[t] W_router^T
// (W_router is [d, N]), plus the token's slot rows of dx in slot order, plus the
// shared experts' dx rows in shared-expert order.  The slot rows of 8 tokens
// are loaded together (a dropped slot reads row 0 and discards it), so that a
// thread keeps 8 loads in flight instead of waiting on each.
constexpr int kDxTok = 8, kDxGroup = 8;
template <bool BF16>
__global__ __launch_bounds__(256) void router_dx_kernel(
    const void* __restrict__ w_router, const float* __restrict__ dlog,
    const float* __restrict__ dx_perm, const int32_t* __restrict__ slot_row,
    const float* __restrict__ dx_shared, int n_shared, int T, int d, int N, int k,
    float* __restrict__ dhidden) {
  extern __shared__ float sh[];          // [kDxTok][N] dlogit, then [kDxTok][k] slot rows
  float* dl = sh;
  int* sr = reinterpret_cast<int*>(sh + kDxTok * N);
  const int t0 = blockIdx.y * kDxTok;
  const int nt = min(kDxTok, T - t0);
  for (int i = threadIdx.x; i < kDxTok * N; i += 256)
    dl[i] = i < nt * N ? dlog[(size_t)t0 * N + i] : 0.f;
  for (int i = threadIdx.x; i < kDxTok * k; i += 256)
    sr[i] = i < nt * k ? slot_row[(size_t)t0 * k + i] : -1;
  __syncthreads();
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (c >= d) return;
  float4 acc[kDxTok];
#pragma unroll
  for (int t = 0; t < kDxTok; ++t) acc[t] = make_float4(0.f, 0.f, 0.f, 0.f);
  auto w_at = [&](int i, int e) {
    return BF16 ? bf16_to_f32(static_cast<const uint16_t*>(w_router)[(size_t)(c + i) * N + e])
                : static_cast<const float*>(w_router)[(size_t)(c + i) * N + e];
  };
  auto fma_e = [&](int e, const float (&wv)[4]) {
#pragma unroll
    for (int t = 0; t < kDxTok; ++t) {
      const float g = dl[t * N + e];
      acc[t].x = fmaf(g, wv[0], acc[t].x);
      acc[t].y = fmaf(g, wv[1], acc[t].y);
      acc[t].z = fmaf(g, wv[2], acc[t].z);
      acc[t].w = fmaf(g, wv[3], acc[t].w);
    }
  };
  // experts in order; the weights of 8 experts are loaded before their products
  int e = 0;
  for (; e + 8 <= N; e += 8) {
    float wv[8][4];
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) wv[q][i] = w_at(i, e + q);
#pragma unroll
    for (int q = 0; q < 8; ++q) fma_e(e + q, wv[q]);
  }
  for (; e < N; ++e) {
    float wv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[i] = w_at(i, e);
    fma_e(e, wv);
  }
#pragma unroll
  for (int t0g = 0; t0g < kDxTok; t0g += kDxGroup) {
    for (int j = 0; j < k; ++j) {
      float4 v[kDxGroup];
#pragma unroll
      for (int t = 0; t < kDxGroup; ++t) {
        const int r = sr[(t0g + t) * k + j];
        v[t] = *reinterpret_cast<const float4*>(dx_perm + (size_t)max(r, 0) * d + c);
      }
#pragma unroll
      for (int t = 0; t < kDxGroup; ++t) {
        if (sr[(t0g + t) * k + j] >= 0) {
          float4& a = acc[t0g + t];
          a.x += v[t].x; a.y += v[t].y; a.z += v[t].z; a.w += v[t].w;
        }
      }
    }
    for (int q = 0; q < n_shared; ++q) {
#pragma unroll
      for (int t = 0; t < kDxGroup; ++t) {
        if (t0g + t < nt) {
          const float4 v = *reinterpret_cast<const float4*>(
              dx_shared + ((size_t)q * T + t0 + t0g + t) * d + c);
          float4& a = acc[t0g + t];
          a.x += v.x; a.y += v.y; a.z += v.z; a.w += v.w;
        }
      }
    }
#pragma unroll
    for (int t = 0; t < kDxGroup; ++t)
      if (t0g + t < nt)
        *reinterpret_cast<float4*>(dhidden + (size_t)(t0 + t0g + t) * d + c) = acc[t0g + t];
  }
}

// Partial dW_router = hidden^T dlogit over one chunk of 64 tokens, for 256
// columns (one per thread) and a group of up to EG experts per block (EG = 8
// when N <= 8, else 16), tokens in order (the hidden values of 16 tokens are
// loaded before their products), stored expert-major ([chunk][N][d], coalesced
// over the columns); the first column block also writes the chunk's partial
// dbias.
constexpr int kDwTok = 64;
template <bool BF16, int EG>
__global__ __launch_bounds__(256) void router_dw_kernel(const void* __restrict__ hidden,
                                                        const float* __restrict__ dlog, int T,
                                                        int d, int N, float* __restrict__ part_w,
                                                        float* __restrict__ part_b) {
  __shared__ float4 dl[kDwTok][EG / 4];
  const int chunk = blockIdx.y, eg = blockIdx.z * EG;
  const int t0 = chunk * kDwTok, nt = min(kDwTok, T - t0);
  const int ne = min(EG, N - eg);
  float* dls = reinterpret_cast<float*>(dl);
  for (int i = threadIdx.x; i < kDwTok * EG; i += 256) {
    const int t = i / EG, e = i % EG;
    dls[i] = (t < nt && e < ne) ? dlog[(size_t)(t0 + t) * N + eg + e] : 0.f;
  }
  __syncthreads();
  if (blockIdx.x == 0 && (int)threadIdx.x < ne) {
    float s = 0.f;
    for (int t = 0; t < nt; ++t) s += dls[t * EG + threadIdx.x];
    part_b[(size_t)chunk * N + eg + threadIdx.x] = s;
  }
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= d) return;
  float acc[EG];
#pragma unroll
  for (int e = 0; e < EG; ++e) acc[e] = 0.f;
  for (int tb = 0; tb < nt; tb += 16) {
    float hv[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int t = min(tb + u, nt - 1);            // rows past the chunk: dl is 0 there
      hv[u] = BF16 ? bf16_to_f32(static_cast<const uint16_t*>(hidden)[(size_t)(t0 + t) * d + c])
                   : static_cast<const float*>(hidden)[(size_t)(t0 + t) * d + c];
    }
#pragma unroll
    for (int u = 0; u < 16; ++u)
#pragma unroll
      for (int e4 = 0; e4 < EG / 4; ++e4) {
        const float4 g = dl[tb + u][e4];
        acc[4 * e4 + 0] = fmaf(hv[u], g.x, acc[4 * e4 + 0]);
        acc[4 * e4 + 1] = fmaf(hv[u], g.y, acc[4 * e4 + 1]);
        acc[4 * e4 + 2] = fmaf(hv[u], g.z, acc[4 * e4 + 2]);
        acc[4 * e4 + 3] = fmaf(hv[u], g.w, acc[4 * e4 + 3]);
      }
  }
#pragma unroll
  for (int e = 0; e < EG; ++e)
    if (e < ne) part_w[((size_t)chunk * N + eg + e) * d + c] = acc[e];
}

// Sum of the chunk partials in a fixed order (deterministic): a block owns 256
// consecutive elements of the expert-major partials (4 columns of one expert per
// lane, 16-byte loads); wave g sums the chunks of its contiguous eighth of the
// chunk range in chunk order, then the eight wave sums are added in wave order
// and written to dW_router [d, N].  The first N threads of block 0 sum dbias in
// chunk order.
constexpr int kDwRedWaves = 8;
__global__ __launch_bounds__(64 * kDwRedWaves) void router_dw_reduce_kernel(
    const float* __restrict__ part_w, const float* __restrict__ part_b, int n_chunks, int d,
    int N, float* __restrict__ dw, float* __restrict__ dbias) {
  __shared__ float4 red[kDwRedWaves][64];
  const int lane = threadIdx.x & 63, g = threadIdx.x >> 6;
  const size_t dn = (size_t)d * N;                      // a multiple of 4
  const size_t i = ((size_t)blockIdx.x * 64 + lane) * 4;  // expert i / d, columns i % d ..
  const int q0 = g * n_chunks / kDwRedWaves, q1 = (g + 1) * n_chunks / kDwRedWaves;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  if (i < dn) {
    int q = q0;
    for (; q + 8 <= q1; q += 8) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const float4*>(part_w + (size_t)(q + u) * dn + i);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        s.x += v[u].x; s.y += v[u].y; s.z += v[u].z; s.w += v[u].w;
      }
    }
    for (; q < q1; ++q) {
      const float4 v = *reinterpret_cast<const float4*>(part_w + (size_t)q * dn + i);
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
  }
  red[g][lane] = s;
  __syncthreads();
  if (g == 0 && i < dn) {
    float4 t = red[0][lane];
#pragma unroll
    for (int w = 1; w < kDwRedWaves; ++w) {
      const float4 v = red[w][lane];
      t.x += v.x; t.y += v.y; t.z += v.z; t.w += v.w;
    }
    const int e = (int)(i / d), c = (int)(i % d);
    dw[(size_t)c * N + e] = t.x;
    dw[(size_t)(c + 1) * N + e] = t.y;
    dw[(size_t)(c + 2) * N + e] = t.z;
    dw[(size_t)(c + 3) * N + e] = t.w;
  }
  if (dbias && blockIdx.x == 0 && (int)threadIdx.x < N) {
    float sb = 0.f;
    for (int q = 0; q < n_chunks; ++q) sb += part_b[(size_t)q * N + threadIdx.x];
    dbias[threadIdx.x] = sb;
  }
}

static int round8(int x) { return (x + 7) & ~7; }

static size_t pad256(size_t b) { return (b + 255) & ~(size_t)255; }

__global__ void zero_i32_kernel(int32_t* __restrict__ q, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) q[i] = 0;
}

// Workspace of the dx GEMM's k-split: one fp32 256 x 256 partial tile and one
// ticket per compute unit (0 bytes without a device, e.g. on a CPU-only host).
size_t split_ws_bytes() {
  const int cus = device_cus();
  if (cus <= 0) return 0;
  return pad256((size_t)cus * kBM * kBN * sizeof(float)) + pad256((size_t)cus * sizeof(int32_t));
}

// Point the dx GEMM's arguments at the split workspace that starts at `base`.
void set_split(Args& s, void* base) {
  const int cus = device_cus();
  if (cus <= 0 || !base) return;
  s.part = static_cast<float*>(base);
  s.tickets = reinterpret_cast<int32_t*>(static_cast<char*>(base) +
                                         pad256((size_t)cus * kBM * kBN * sizeof(float)));
  s.num_cus = cus;
}

template <int MODE>
static void gemm(const Args& a, bool bf16, hipStream_t stream) {
  if (bf16) {
    Args b = a;
    b.n_tiles = a.Nn / (MODE == kSwiGLU ? kBN / 2 : kBN);
    int grid;
    if (MODE == kWGrad) {
      grid = round8((a.M / kBM) * b.n_tiles * a.n_exp);
    } else {
      const int mt_bound = (a.max_rows + kBM - 1) / kBM + a.n_exp;
      grid = round8(mt_bound * b.n_tiles);
    }
    b.dp_grid = grid;
    if (MODE == kDX && a.tickets) {
      hipLaunchKernelGGL(zero_i32_kernel, dim3((a.num_cus + 255) / 256), dim3(256), 0, stream,
                         a.tickets, a.num_cus);
      grid += round8(a.num_cus);
    }
    hipLaunchKernelGGL(bwd_gemm_bf16_kernel<MODE>, dim3(grid), dim3(kThreads), 0, stream, b);
  } else {
    Args b = a;
    b.n_tiles = a.Nn / kFB;
    dim3 grid;
    if (MODE == kWGrad) grid = dim3(a.M / kFB, b.n_tiles, a.n_exp);
    else grid = dim3((a.max_rows + kFB - 1) / kFB + a.n_exp, b.n_tiles, 1);
    hipLaunchKernelGGL(bwd_gemm_f32_kernel<MODE>, grid, dim3(256), 0, stream, b);
  }
}

}  // namespace bwd

size_t expert_backward_ws_bytes(int d, int f, int max_rows, bool bf16) {
  (void)d;
  const size_t rows = (size_t)max_rows, eb = bf16 ? 2 : 4;
  return bwd::pad256(rows * f * 4) + bwd::pad256(rows * 2 * f * eb) + bwd::pad256(rows * f * eb) +
         (bf16 ? bwd::split_ws_bytes() : 0);
}

hipError_t launch_combine_backward(const void* dy, const float* y_perm, const int32_t* slot_row,
                                   const float* topk_w, int T, int d, int k, bool bf16,
                                   void* g_perm, float* dgate, hipStream_t stream) {
  const dim3 grid((T + 3) / 4);
  if (bf16)
    hipLaunchKernelGGL(bwd::combine_bwd_kernel<true>, grid, dim3(256), 0, stream, dy, y_perm,
                       slot_row, topk_w, T, d, k, g_perm, dgate);
  else
    hipLaunchKernelGGL(bwd::combine_bwd_kernel<false>, grid, dim3(256), 0, stream, dy, y_perm,
                       slot_row, topk_w, T, d, k, g_perm, dgate);
  return hipGetLastError();
}

hipError_t launch_expert_backward(const void* x_perm, const void* g_perm, const int32_t* offsets,
                                  const void* w1, const void* w3, const void* w2, int N, int d,
                                  int f, int max_rows, bool bf16, float* dx_perm, float* dw1,
                                  float* dw3, float* dw2, void* ws, hipStream_t stream) {
  using namespace bwd;
  const size_t rows = (size_t)max_rows, eb = bf16 ? 2 : 4;
  char* base = static_cast<char*>(ws);
  float* da = reinterpret_cast<float*>(base);
  void* dh = base + pad256(rows * f * 4);
  void* act = static_cast<char*>(dh) + pad256(rows * 2 * f * eb);
  Args a{};
  a.offsets = offsets;
  a.n_exp = N;
  a.max_rows = max_rows;

  // da = g W2_e^T  ([rows, d] x [f, d]^T)
  Args s = a;
  s.a = g_perm; s.lda = d;
  s.b0 = w2; s.b1 = w2; s.ldb = d; s.b_estride = (long long)f * d;
  s.K = d; s.Nn = f; s.out0 = da; s.ldo = f;
  gemm<kDA>(s, bf16, stream);

  // recompute h1, h3 and form dh1, dh3, a
  s = a;
  s.a = x_perm; s.lda = d;
  s.b0 = w1; s.b1 = w3; s.ldb = f; s.b_estride = (long long)d * f;
  s.K = d; s.Nn = f; s.da = da; s.dh = dh; s.act = act; s.f = f;
  gemm<kSwiGLU>(s, bf16, stream);

  // dx = [dh1 | dh3] [W1_e | W3_e]^T  ([rows, 2f] x [d, 2f]^T)
  s = a;
  s.a = dh; s.lda = 2 * f;
  s.b0 = w1; s.b1 = w3; s.ldb = f; s.b_estride = (long long)d * f;
  s.K = 2 * f; s.ksplit = f / kBK; s.Nn = d; s.out0 = dx_perm; s.ldo = d;
  if (bf16) set_split(s, static_cast<char*>(act) + pad256(rows * f * eb));
  gemm<kDX>(s, bf16, stream);

  // dW2_e = a_e^T g_e  ([f, rows] x [rows, d])
  s = a;
  s.a = act; s.lda = f;
  s.b0 = g_perm; s.b1 = g_perm; s.ldb = d;
  s.M = f; s.Nn = d; s.out0 = dw2; s.out1 = dw2; s.ldo = d; s.nsplit = d;
  s.o_estride = (long long)f * d;
  gemm<kWGrad>(s, bf16, stream);

  // [dW1_e | dW3_e] = x_e^T [dh1_e | dh3_e]  ([d, rows] x [rows, 2f])
  s = a;
  s.a = x_perm; s.lda = d;
  s.b0 = dh; s.b1 = dh; s.ldb = 2 * f;
  s.M = d; s.Nn = 2 * f; s.out0 = dw1; s.out1 = dw3; s.ldo = f; s.nsplit = f;
  s.o_estride = (long long)d * f;
  gemm<kWGrad>(s, bf16, stream);
  return hipGetLastError();
}

size_t expert_backward_saved_ws_bytes(int d, int f, int max_rows, bool bf16) {
  (void)d;
  const size_t rows = (size_t)max_rows, eb = bf16 ? 2 : 4;
  return bwd::pad256(rows * 2 * f * eb) + bwd::pad256(rows * f * eb) +
         (bf16 ? bwd::split_ws_bytes() : 0);
}

hipError_t launch_expert_backward_saved(const void* x_perm, const void* g_perm, const void* h13,
                                        const void* act_in, const int32_t* offsets,
                                        const void* w1, const void* w3,
                                        const void* w2, int N, int d, int f, int max_rows,
                                        bool bf16, float* dx_perm, float* dw1, float* dw3,
                                        float* dw2, void* ws, hipStream_t stream) {
  using namespace bwd;
  const size_t rows = (size_t)max_rows, eb = bf16 ? 2 : 4;
  void* dh = ws;
  // the forward's activations when the caller has them, else recomputed here
  void* act_ws = static_cast<char*>(ws) + pad256(rows * 2 * f * eb);
  const void* act = act_in ? act_in : act_ws;
  Args a{};
  a.offsets = offsets;
  a.n_exp = N;
  a.max_rows = max_rows;

  // da = g W2_e^T, and in the same epilogue dh1, dh3, a from the saved h1 / h3
  Args s = a;
  s.a = g_perm; s.lda = d;
  s.b0 = w2; s.b1 = w2; s.ldb = d; s.b_estride = (long long)f * d;
  s.K = d; s.Nn = f; s.h13 = h13; s.dh = dh; s.act = act_in ? nullptr : act_ws; s.f = f;
  gemm<kDAS>(s, bf16, stream);

  // dx = [dh1 | dh3] [W1_e | W3_e]^T
  s = a;
  s.a = dh; s.lda = 2 * f;
  s.b0 = w1; s.b1 = w3; s.ldb = f; s.b_estride = (long long)d * f;
  s.K = 2 * f; s.ksplit = f / kBK; s.Nn = d; s.out0 = dx_perm; s.ldo = d;
  if (bf16) set_split(s, static_cast<char*>(act_ws) + pad256(rows * f * eb));
  gemm<kDX>(s, bf16, stream);

  // dW2_e = a_e^T g_e
  s = a;
  s.a = act; s.lda = f;
  s.b0 = g_perm; s.b1 = g_perm; s.ldb = d;
  s.M = f; s.Nn = d; s.out0 = dw2; s.out1 = dw2; s.ldo = d; s.nsplit = d;
  s.o_estride = (long long)f * d;
  gemm<kWGrad>(s, bf16, stream);

  // [dW1_e | dW3_e] = x_e^T [dh1_e | dh3_e]
  s = a;
  s.a = x_perm; s.lda = d;
  s.b0 = dh; s.b1 = dh; s.ldb = 2 * f;
  s.M = d; s.Nn = 2 * f; s.out0 = dw1; s.out1 = dw3; s.ldo = f; s.nsplit = f;
  s.o_estride = (long long)d * f;
  gemm<kWGrad>(s, bf16, stream);
  return hipGetLastError();
}

size_t router_backward_ws_bytes(int T, int d, int N) {
  const size_t chunks = (size_t)(T + bwd::kDwTok - 1) / bwd::kDwTok;
  return bwd::pad256((size_t)T * N * 4) + bwd::pad256(chunks * d * N * 4) +
         bwd::pad256(chunks * N * 4);
}

hipError_t launch_router_backward(const void* hidden, const void* w_router, const float* logits,
                                  const int32_t* topk_idx, const float* topk_w,
                                  const int32_t* counts, const float* dgate, const float* dx_perm,
                                  const int32_t* slot_row, const float* dx_shared, int n_shared,
                                  float aux_coef, int T, int d, int N, int k, bool bf16,
                                  float* dhidden, float* dw_router, float* dbias, void* ws,
                                  hipStream_t stream) {
  using namespace bwd;
  const int chunks = (T + kDwTok - 1) / kDwTok;
  char* base = static_cast<char*>(ws);
  float* dlog = reinterpret_cast<float*>(base);
  float* part_w = reinterpret_cast<float*>(base + pad256((size_t)T * N * 4));
  float* part_b = reinterpret_cast<float*>(reinterpret_cast<char*>(part_w) +
                                           pad256((size_t)chunks * d * N * 4));
  hipLaunchKernelGGL(router_dlogit_kernel, dim3((T + 255) / 256), dim3(256), 0, stream, logits,
                     topk_idx, topk_w, counts, dgate, aux_coef, T, N, k, dlog);
  const dim3 gx((d + 1023) / 1024, (T + kDxTok - 1) / kDxTok);
  const size_t shx = (size_t)kDxTok * (N + k) * 4;
  if (bf16)
    hipLaunchKernelGGL(router_dx_kernel<true>, gx, dim3(256), shx, stream, w_router, dlog, dx_perm,
                       slot_row, dx_shared, n_shared, T, d, N, k, dhidden);
  else
    hipLaunchKernelGGL(router_dx_kernel<false>, gx, dim3(256), shx, stream, w_router, dlog,
                       dx_perm, slot_row, dx_shared, n_shared, T, d, N, k, dhidden);
  const int eg_w = N <= 8 ? 8 : 16;
  const dim3 gw((d + 255) / 256, chunks, (N + eg_w - 1) / eg_w);
  if (bf16 && eg_w == 8)
    hipLaunchKernelGGL((router_dw_kernel<true, 8>), gw, dim3(256), 0, stream, hidden, dlog, T, d,
                       N, part_w, part_b);
  else if (bf16)
    hipLaunchKernelGGL((router_dw_kernel<true, 16>), gw, dim3(256), 0, stream, hidden, dlog, T, d,
                       N, part_w, part_b);
  else if (eg_w == 8)
    hipLaunchKernelGGL((router_dw_kernel<false, 8>), gw, dim3(256), 0, stream, hidden, dlog, T, d,
                       N, part_w, part_b);
  else
    hipLaunchKernelGGL((router_dw_kernel<false, 16>), gw, dim3(256), 0, stream, hidden, dlog, T,
                       d, N, part_w, part_b);
  const size_t dn = (size_t)d * N;
  hipLaunchKernelGGL(router_dw_reduce_kernel, dim3((unsigned)((dn + 255) / 256)),
                     dim3(64 * kDwRedWaves), 0, stream, part_w, part_b, chunks, d, N, dw_router,
                     dbias);
  return hipGetLastError();
}

}  // namespace moe
