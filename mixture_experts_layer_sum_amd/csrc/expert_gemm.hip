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
// bf16 path (MFMA): a block computes a 256-row x 256-column tile with 8 waves,
// two per SIMD: the SIMDs split the tile 2 x 2 into 128 x 128 quadrants and
// the two waves of a SIMD take 64 columns each (128 x 64 per wave: 8 x 4
// blocks of the 16x16x32 bf16 MFMA, fp32 accumulators), so one wave's MFMAs
// overlap the other's LDS reads and load issue.  Under the chip's power limit
// the 16x16x32 MFMA sustains a higher clock than the 32x32x16 one for the same
// work (an MFMA-only loop on random data measured 1.90 vs 1.75 PFLOP/s); the
// LDS bytes per flop depend on the 128 x 64 wave tile only, not on the MFMA
// shape.  For `up` the 256 columns are 128 columns of W1 and the same 128
// columns of W3, and each wave holds 32 columns of each, so both halves of its
// SwiGLU products are in the same lane.
// k advances 64 at a time (two 32-deep MFMA slices) through two 64 KB LDS
// stages filled by direct buffer -> LDS loads (no VGPRs in flight; every
// request is a whole 128-byte line).  The texture unit accepts these loads at
// about 64 bytes per clock per CU, so a 64 KB stage keeps it busy for about
// half of the stage's MFMA time, and a wave waiting to issue a load cannot
// issue MFMAs.  Only one wave of each SIMD loads (16 instructions per stage,
// one per two MFMAs of the slice that follows the barrier); the other wave
// only computes and keeps the matrix core busy meanwhile.
// A (x_perm rows) is stored row-major and read with ds_read_b128; the
// weights stay n-contiguous in LDS and the MFMA B operand (8 consecutive k per
// lane) is assembled with the gfx950 transposing read ds_read_b64_tr_b16.
// Both LDS layouts are XOR-swizzled per row (the weights' also padded every
// four k-rows) so that the fragment reads are bank-conflict free.  One
// barrier per k-step, placed after the last fragment read of the current
// stage: the stage is refilled two steps ahead while the second slice's MFMAs
// run.
// A wave's four 32-row sub-tiles are tile rows 32 (2i + wm) (the two row
// halves interleave), so in an expert's last, partial tile both halves have
// about the same number of real rows; sub-tiles with no real row skip their
// fragment reads and MFMAs (the loop is instantiated per count).  Rows past
// the tile's end lie past the range of the A buffer resource and load as
// zeros.
// The row tiles of all experts are numbered consecutively; a block finds its
// expert with a wave-wide prefix scan of the per-expert tile counts read from
// `offsets` on the device, so the host never needs the routing result.
// Blocks are dealt round-robin to the 8 XCDs; each XCD gets a contiguous range
// of the real tiles, walked 8 row tiles at a time per column tile, so the
// blocks an XCD runs together share A rows and weight columns in its L2.
#include <atomic>

#include "common.hpp"
#include "internal.hpp"

namespace moe {

constexpr int kBM = 256, kBN = 256, kGemmThreads = 512;
constexpr int kGroupM = 8;


// Data-parallel block -> logical tile.  Blocks are dealt round-robin to the 8
// XCDs, so block b runs on XCD b % 8: give XCD x the contiguous range
// [x*per, (x+1)*per) of the `total` logical tiles (per = ceil(total / 8)).
__device__ __forceinline__ bool dp_logical(int total, int& logical) {
  const int per = (total + 7) >> 3;
  const int b = blockIdx.x;
  const int local = b >> 3;
  if (local >= per) return false;
  logical = (b & 7) * per + local;
  return logical < total;
}

// Logical tile -> (row tile, column tile): kGroupM row tiles are walked for
// every column tile, so the blocks an XCD runs at the same time share A rows
// and weight columns in its L2.
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

// Row tile `mt` of the 256-row tiling, with each expert's rows spread evenly
// over its ceil(R / 256) tiles in whole 64-row units (R rows = u units; every
// tile gets floor(u / n) or one more), so that no tile is a sliver: a tile's
// cost follows its 64-row blocks only while the matrix cores bound it, and a
// tile of a few rows costs nearly a full one (it still streams its whole
// weight slice).  rend is the tile's own end.  Wave-uniform.
__device__ __forceinline__ bool find_tile_balanced(const int32_t* __restrict__ offsets, int N,
                                                   int mt, int max_rows, int& e_out, int& r0,
                                                   int& rend) {
  int e, t0, t1;
  if (!find_tile(offsets, N, mt, kBM, max_rows, e, t0, t1)) return false;
  const int o0 = min(max(offsets[e], 0), max_rows);
  const int R = t1 - o0;                       // the expert's rows (t1 is its end)
  const int j = (t0 - o0) / kBM;               // tile index within the expert
  const int n = (R + kBM - 1) / kBM, u = (R + 63) / 64;
  const int q = u / n, rem = u - q * n;
  const int start = 64 * (j * q + min(j, rem));
  const int size = 64 * (q + (j < rem ? 1 : 0));
  e_out = e;
  r0 = o0 + start;
  rend = min(o0 + start + size, t1);
  return true;
}

// Heaviest-first order of the balanced row tiles.  A balanced tile holds 1..4
// units of 64 rows (an expert with R rows has n = ceil(R / 256) tiles and
// u = ceil(R / 64) units: its first u % n tiles hold floor(u / n) + 1 units,
// the rest floor(u / n)).  When the grid is short and the tiles differ,
// dispatching them in order of units (4 first; ties by expert, then tile)
// lets the CUs that finish a lighter tile early take the next light one
// instead of the grid ending on a round of heavy tiles, and dealing tile b to
// XCD b % 8 spreads the heavy tiles evenly over the XCDs (the grouped order
// hands whole groups of row tiles to one XCD).  Measured: skewed routing with
// re-routing (36 experts, 992 tiles) up 461 -> 437 us, down 244 -> 239 us;
// 16 experts with K = 5632 (304 down tiles) 277 -> 267 us.  A light tile
// costs nearly as much as a full one (its two-stage load pipeline waits on
// memory latency either way), so 16 skewed experts with 416 tiles gain nothing.
//
// lpt_classes: the number of row tiles of each weight w = 1..4 (cls[w - 1]).
__device__ __forceinline__ void lpt_classes(const int32_t* __restrict__ offsets, int N,
                                            int max_rows, int (&cls)[4]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int w = 0; w < 4; ++w) cls[w] = 0;
  for (int b = 0; b < N; b += 64) {
    const int e = b + lane;
    int c[4] = {0, 0, 0, 0};
    if (e < N) {
      const int o0 = min(max(offsets[e], 0), max_rows);
      const int o1 = min(max(offsets[e + 1], o0), max_rows);
      const int R = o1 - o0;
      if (R > 0) {
        const int n = (R + kBM - 1) / kBM, u = (R + 63) / 64;
        const int q = u / n, rem = u - q * n;
#pragma unroll
        for (int w = 1; w <= 4; ++w) c[w - 1] = (q + 1 == w ? rem : 0) + (q == w ? n - rem : 0);
      }
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      int v = c[w];
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
      cls[w] += v;
    }
  }
}

// Row tile number s of the heaviest-first order (cls from lpt_classes): its
// expert and rows [r0, rend), the same rows find_tile_balanced gives that tile.
__device__ __forceinline__ bool find_tile_lpt(const int32_t* __restrict__ offsets, int N, int s,
                                              int max_rows, const int (&cls)[4], int& e_out,
                                              int& r0, int& rend) {
  int w = 4;
  while (w > 0 && s >= cls[w - 1]) {
    s -= cls[w - 1];
    --w;
  }
  if (w == 0) return false;
  const int lane = threadIdx.x & 63;
  int before = 0;
  for (int b = 0; b < N; b += 64) {
    const int e = b + lane;
    int o0 = 0, o1 = 0, q = 0, rem = 0, cnt = 0;
    if (e < N) {
      o0 = min(max(offsets[e], 0), max_rows);
      o1 = min(max(offsets[e + 1], o0), max_rows);
      const int R = o1 - o0;
      if (R > 0) {
        const int n = (R + kBM - 1) / kBM, u = (R + 63) / 64;
        q = u / n;
        rem = u - q * n;
        cnt = (q + 1 == w ? rem : 0) + (q == w ? n - rem : 0);
      }
    }
    int inc = cnt;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const int v = __shfl_up(inc, m, 64);
      if (lane >= m) inc += v;
    }
    const int tot = __shfl(inc, 63, 64);
    if (s < before + tot) {
      const unsigned long long bal = __ballot(before + inc > s);
      const int L = __ffsll(static_cast<long long>(bal)) - 1;
      const int idx = s - before - __shfl(inc - cnt, L, 64);
      const int qL = __shfl(q, L, 64), remL = __shfl(rem, L, 64), oL = __shfl(o0, L, 64);
      const int j = (w == qL + 1 ? 0 : remL) + idx;          // tile within the expert
      const int start = 64 * (j * qL + min(j, remL));
      e_out = b + L;
      r0 = oL + start;
      rend = min(oL + start + 64 * (qL + (j < remL ? 1 : 0)), __shfl(o1, L, 64));
      return true;
    }
    before += tot;
  }
  return false;
}

// Heaviest-first dispatch is used when some row tile is light and the grid
// is at most this many rounds of the CUs; longer grids keep the grouped,
// XCD-contiguous order, whose L2 reuse matters more than the last round
// (16 experts, K = 2048, 1672 tiles: 390 us grouped, 404 us heaviest-first;
// Mixtral counts, 7504 tiles: 3.09 ms grouped, 3.20 ms heaviest-first).
constexpr int kLptRounds = 4;

// Split of the last, partial round of tiles over k.  With `total` tiles on
// `num_cus` CUs (one block each) the last round holds r = total % num_cus
// tiles; when that round would leave at least half of the CUs idle, each of
// its r tiles is cut into `segs` k-ranges run by separate blocks (segs <= 4,
// each range at least two k-steps).  Returns the number of tiles computed
// whole (the first n_dp logical tiles).  Only deep tiles are split: the few
// CUs of an unsplit last round run at a much higher clock under the chip's
// power limit, so for K = 5632 (88 k-steps, 48 tail tiles) the whole tiles
// finished sooner (272 us) than four ranges each (331 us), while for
// K = 14336 (224 k-steps, the same 48 tail tiles) the split won (1671 against
// 1780 us).
constexpr int kMaxSegs = 4;
constexpr int kMinSplitSteps = 128;
__device__ __forceinline__ int split_plan(int total, int nk, int num_cus, int& segs) {
  segs = 1;
  if (num_cus <= 0 || nk < kMinSplitSteps) return total;
  const int r = total % num_cus;
  if (r == 0 || 2 * r > num_cus) return total;
  int s = num_cus / r;
  s = s < kMaxSegs ? s : kMaxSegs;
  s = s < nk / 2 ? s : nk / 2;
  if (s < 2) return total;
  segs = s;
  return total - r;
}

typedef int i32x4 __attribute__((ext_vector_type(4)));
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9 family)

__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kBK = 64;
// B half of a stage: per 128-column sub-tile, 16 groups of 4 k-rows (the 1 KB
// that one load instruction writes) each followed by 16 bytes of padding.
constexpr int kBGroup = 4 * 128 + 8, kBSub = 16 * kBGroup, kStage = 16384 + 2 * kBSub;

// Direct global -> LDS loads of one 64-deep k-step into the stage at `dst`:
// A at element 0, B sub-tile q at 16384 + kBSub q.  Only the four waves
// w = 0..3 load (8 A and 8 B instructions each).
struct LoadState {
  uint32_t a_v0, a_v1, b_v;     // per-lane parts of the A (row parity 0 / 1) and B offsets
  uint32_t a_u, b_u;            // wave-uniform parts
  uint32_t a_step, b_step;      // bytes between this wave's consecutive A / B instructions
};
__device__ __forceinline__ void gemm_issue(uint16_t* __restrict__ dst, __amdgpu_buffer_rsrc_t a_rs,
                                           __amdgpu_buffer_rsrc_t b_rs, const LoadState& L, int w,
                                           int kstep, int Nout) {
  const uint32_t ka = (uint32_t)kstep * (kBK * 2);
  const uint32_t kb = (uint32_t)kstep * (uint32_t)(kBK * Nout * 2);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rs, (lds_void*)(dst + (8 * w + i) * 512), 16,
                                             ((i & 1) ? L.a_v1 : L.a_v0) + (L.a_u + i * L.a_step + ka), 0, 0, 0);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rs, (lds_void*)(dst + 16384 + kBSub * (w >> 1) +
                                                               kBGroup * (8 * (w & 1) + i)), 16,
                                             L.b_v + (L.b_u + i * L.b_step + kb), 0, 0, 0);
}


// Fragments of the 16x16x32 MFMA (lane l: row / column l % 16, k values
// 8 (l / 16) .. +7 of a 32-deep slice).  A row block ib of slice s is one
// ds_read_b128 at a_base[s] + 4096 (ib / 2) + 1024 (ib % 2); B column block
// jb = 2 j + jj is two transposing reads at b_base[j] + 16 jj + 8 kBGroup s
// (k rows +0..3 and, one padded group later, +4..7 of the lane group).
__device__ __forceinline__ uint4 rd_b(const uint16_t* __restrict__ st, int b_addr) {
  const uint16_t* p = st + 16384 + b_addr;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p + kBGroup));
  const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
  return make_uint4(l2.x, l2.y, h2.x, h2.y);
}

__device__ __forceinline__ uint4 rd_a(const uint16_t* __restrict__ st, int a_addr, int ib) {
  return *reinterpret_cast<const uint4*>(st + a_addr + 4096 * (ib >> 1) + 1024 * (ib & 1));
}

__device__ __forceinline__ void rd_bs(const uint16_t* __restrict__ st, const int (&b_base)[2], int s,
                                      uint4 (&fb)[4]) {
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) fb[jb] = rd_b(st, b_base[jb >> 1] + 16 * (jb & 1) + 8 * kBGroup * s);
}

// The 32 MFMAs of one slice for the NB row blocks that hold rows (A in fa, B
// in fb).  Each A register is refilled with the next slice's fragment (slice
// ns of stage nst) right after its last use; with ROLLB the B registers are
// refilled the same way during the last row block (fewer registers live),
// otherwise the caller reads the next B into registers of its own first.
template <int NB, bool ROLLB>
__device__ __forceinline__ void slice_mma(uint4 (&fb)[4], uint4 (&fa)[8], f32x4 (&acc)[8][4],
                                          const uint16_t* __restrict__ nst, const int (&a_base)[2],
                                          const int (&b_base)[2], int ns) {
#pragma unroll
  for (int ib = 0; ib < NB; ++ib) {
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      acc[ib][jb] = mfma16(fa[ib], fb[jb], acc[ib][jb]);
      if (ROLLB && ib == NB - 1) fb[jb] = rd_b(nst, b_base[jb >> 1] + 16 * (jb & 1) + 8 * kBGroup * ns);
    }
    fa[ib] = rd_a(nst, a_base[ns], ib);
  }
}

// Wait until this wave's LDS reads are done and all of its direct loads have
// landed, then meet the other waves.  One asm statement with a memory clobber
// (no load in it), so that no LDS access moves across it.
#define MOE_WAIT_BARRIER() asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory")

// One 64-deep k-step (two 32-deep slices).  On entry fa/fb hold slice 0 of
// stage `cur`.  The barrier after the last fragment read of `cur` certifies
// that every wave is done with it and that the next step has landed in `nxt`;
// `cur` is then refilled two steps ahead while slice 1's MFMAs run, and the
// next step's slice 0 is read from `nxt`.  `dst` is `cur`: a separate restrict
// parameter only so that the refill carries its own alias scope and reading
// `nxt` does not wait for it.
template <int NB, bool DMA, bool ROLLB>
__device__ __forceinline__ void gemm_step(const uint16_t* __restrict__ cur, uint16_t* __restrict__ dst,
                                          const uint16_t* __restrict__ nxt,
                                          __amdgpu_buffer_rsrc_t a_rs, __amdgpu_buffer_rsrc_t b_rs,
                                          const LoadState& Ld, int w, int kstep, int Nout,
                                          const int (&a_base)[2], const int (&b_base)[2],
                                          f32x4 (&acc)[8][4], uint4 (&fa)[8], uint4 (&fb)[4]) {
  uint4 fb1[4];
  if (NB > 0) {
    if (ROLLB) {
      slice_mma<NB, true>(fb, fa, acc, cur, a_base, b_base, 1);
    } else {
      rd_bs(cur, b_base, 1, fb1);
      slice_mma<NB, false>(fb, fa, acc, cur, a_base, b_base, 1);
      if (NB == 8) {
        // the compute waves as well: the next slice's B first, then one A refill
        // after each row block's MFMAs (left alone, the scheduler reads some A
        // blocks just before their MFMAs and waits for them)
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  MOE_WAIT_BARRIER();
  if (DMA && NB == 8) {
    // the refill is interleaved with slice 1's MFMAs, one load per two MFMAs,
    // so that this wave's MFMAs run while it waits to issue its loads
    if (ROLLB) {
      gemm_issue(dst, a_rs, b_rs, Ld, w, kstep, Nout);
      slice_mma<NB, true>(fb, fa, acc, nxt, a_base, b_base, 0);
#pragma unroll
      for (int i = 0; i < 7; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 9, 0);
    } else {
      rd_bs(nxt, b_base, 0, fb);
      gemm_issue(dst, a_rs, b_rs, Ld, w, kstep, Nout);
      slice_mma<NB, false>(fb1, fa, acc, nxt, a_base, b_base, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  } else {
    if (DMA) gemm_issue(dst, a_rs, b_rs, Ld, w, kstep, Nout);
    __builtin_amdgcn_sched_barrier(0);     // keep the refill right after the barrier
    if (NB > 0) {
      if (ROLLB) {
        slice_mma<NB, true>(fb, fa, acc, nxt, a_base, b_base, 0);
      } else {
        rd_bs(nxt, b_base, 0, fb);
        slice_mma<NB, false>(fb1, fa, acc, nxt, a_base, b_base, 0);
        if (NB == 8) {
          __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }
}

// LDS layout of one stage (kStage elements, 64.5 KB):
//   A  [256 rows][64 k]   rows of 8 x 16-byte chunks (one full 128-byte line
//                          of x_perm per row); chunk c of row r sits at
//                          position c ^ ((r >> 1) & 7)
//   B  2 sub-tiles [64 k][128 n], rows of 16 chunks; chunk c of row k sits at
//                          position c ^ (4 * (k & 3)); every 4 k-rows (the 1 KB
//                          one load instruction writes) are followed by 16
//                          bytes of padding
// The A swizzle makes its reads conflict-free.  A 32-lane half of a transposing
// B read covers k rows r .. r+3 and r+8 .. r+11, which share their swizzle; the
// padding shifts the second group of rows by two 16-byte bank slots, into the
// slots the first group leaves free.
template <bool UP>
__global__ __launch_bounds__(kGemmThreads, 1) void grouped_gemm_bf16_kernel(
    const uint16_t* __restrict__ X, const int32_t* __restrict__ offsets, int N,
    const uint16_t* __restrict__ Wa, const uint16_t* __restrict__ Wb, int K, int Nout,
    int n_tiles, int max_rows, void* __restrict__ out, float* __restrict__ part,
    int32_t* __restrict__ tickets, int num_cus, int dp_grid, uint16_t* __restrict__ h13) {
  // two 64 KB stages as separate LDS objects: the compiler tracks in-flight
  // direct loads per LDS object, so a read of one stage never waits on the
  // refill of the other
  __shared__ __align__(1024) uint16_t S0[kStage], S1[kStage];
  __shared__ int s_last;

  const int nk = K / kBK;
  int cls[4];
  lpt_classes(offsets, N, max_rows, cls);
  const int m_tiles = cls[0] + cls[1] + cls[2] + cls[3];
  const int total = m_tiles * n_tiles;
  // heaviest-first: block b computes tile b (row tile b / n_tiles of that
  // order, column tile b % n_tiles), so XCD b % 8 gets every eighth tile
  const bool lpt = num_cus > 0 && cls[3] != m_tiles && total <= kLptRounds * num_cus;
  int segs = 1;
  const int n_dp = (UP || lpt || !tickets) ? total : split_plan(total, nk, num_cus, segs);
  // blocks [0, dp_grid) compute whole tiles; the rest compute k-ranges of the
  // last n_sk tiles (block j: tile n_dp + j / segs, range j % segs)
  int logical, kb = 0, kl = nk, slot = -1;
  if ((int)blockIdx.x < dp_grid) {
    if (lpt) {
      logical = blockIdx.x;
      if (logical >= total) return;
    } else if (!dp_logical(n_dp, logical)) {
      return;
    }
  } else {
    const int j = blockIdx.x - dp_grid;
    if (j >= (total - n_dp) * segs) return;
    logical = n_dp + j / segs;
    const int seg = j % segs;
    kb = seg * nk / segs;
    kl = (seg + 1) * nk / segs - kb;
    slot = j;
  }
  kb = __builtin_amdgcn_readfirstlane(kb);
  kl = __builtin_amdgcn_readfirstlane(kl);
  slot = __builtin_amdgcn_readfirstlane(slot);
  int mt, nt, e, r0, rend;
  if (lpt) {
    mt = logical / n_tiles;
    nt = logical - mt * n_tiles;
    if (!find_tile_lpt(offsets, N, mt, max_rows, cls, e, r0, rend)) return;
  } else {
    tile_of_logical(logical, m_tiles, n_tiles, mt, nt);
    if (!find_tile_balanced(offsets, N, mt, max_rows, e, r0, rend)) return;
  }
  e = __builtin_amdgcn_readfirstlane(e);
  r0 = __builtin_amdgcn_readfirstlane(r0);
  rend = __builtin_amdgcn_readfirstlane(rend);
  nt = __builtin_amdgcn_readfirstlane(nt);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sm = w & 3, pw = w >> 2;        // SIMD quadrant, half of it
  const int wm = sm & 1, wn = sm >> 1;
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

  // ---- direct global -> LDS loads: waves 0..3 issue A instructions 8w..8w+7
  // (8 rows each) and B instructions 8w..8w+7 (4 k-rows of sub-tile (8w+i) / 16);
  // waves 4..7 only compute, so on every SIMD one wave keeps issuing MFMAs while
  // the other waits for the texture unit to accept its loads.
  // Rows past the tile's end lie past the A resource's range and load as zeros.
  const int wl = w & 3;
  LoadState Ld;
  {
    const int rl = lane >> 3;                               // row within an 8-row instruction
    Ld.a_v0 = (uint32_t)((rl * K + 8 * ((lane & 7) ^ (lane >> 4))) * 2);
    Ld.a_v1 = (uint32_t)((rl * K + 8 * ((lane & 7) ^ (4 + (lane >> 4)))) * 2);
    Ld.a_u = (uint32_t)(16 * K * 8 * wl);
    Ld.a_step = (uint32_t)(16 * K);
    const int cb = (lane & 15) ^ (4 * (lane >> 4));
    Ld.b_v = (uint32_t)(((lane >> 4) * Nout + 8 * cb) * 2);
    const int colbase = UP ? n0 : n0 + 128 * (wl >> 1);
    Ld.b_u = (uint32_t)((32 * (wl & 1) * Nout + colbase) * 2);
    Ld.b_step = (uint32_t)(8 * Nout);
  }
  const __amdgpu_buffer_rsrc_t b_rs = (wl >> 1) ? b_rs1 : b_rs0;   // wave-uniform

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.f;

  // A: row block ib = rows 64 (ib >> 1) + 32 wm + 16 (ib & 1) + (lane & 15),
  // chunk 4 s + (lane >> 4); the swizzle depends on the lane only
  int a_base[2];
  {
    const int row = 32 * wm + (lane & 15);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) a_base[s2] = row * 64 + 8 * ((4 * s2 + (lane >> 4)) ^ ((row >> 1) & 7));
  }
  // B (transposing read): group gq = lane / 16 covers k rows 8 gq + 4 t .. +3 of the
  // slice; lane i of the group points at row i / 4, columns 4 (i % 4) .. +3
  int b_base[2];
  {
    const int gq = lane >> 4, i16 = lane & 15;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int q = UP ? j : wn;
      const int cb = UP ? (wn * 64 + 32 * pw) : (64 * pw + 32 * j);
      const int col = cb + 4 * (i16 & 3);
      const int kr = 8 * gq + (i16 >> 2);
      const int c = (col >> 3) ^ (4 * (kr & 3));
      b_base[j] = q * kBSub + (kr >> 2) * kBGroup + (kr & 3) * 128 + 8 * c + (col & 7);
    }
  }

  // 32-row sub-tiles of this wave that hold rows of the expert (the rest are
  // padding of the expert's last tile and are skipped)
  const int nv = __builtin_amdgcn_readfirstlane(
      min(4, max(0, (tile_rows - 32 * wm + 63) / 64)));
#define MOE_KLOOP(NV, D0, D1)                                                                   \
  do {                                                                                          \
    uint4 fa[8], fb[4];                                                                         \
    if (2 * NV > 0) {                                                                           \
      rd_bs(S0, b_base, 0, fb);                                                                 \
      _Pragma("unroll") for (int ib = 0; ib < 2 * NV; ++ib) fa[ib] = rd_a(S0, a_base[0], ib);    \
    }                                                                                           \
    int kt = 0;                                                                                 \
    for (; kt + 2 <= kl; kt += 2) {                                                             \
      gemm_step<2 * NV, D0, !UP>(S0, S0, S1, a_rs, b_rs, Ld, wl, kb + min(kt + 2, kl - 1),      \
                                 Nout, a_base, b_base, acc, fa, fb);                            \
      gemm_step<2 * NV, D1, !UP>(S1, S1, S0, a_rs, b_rs, Ld, wl, kb + min(kt + 3, kl - 1),      \
                                 Nout, a_base, b_base, acc, fa, fb);                            \
    }                                                                                           \
    if (kt < kl)                                                                                \
      gemm_step<2 * NV, D0, !UP>(S0, S0, S1, a_rs, b_rs, Ld, wl, kb + min(kt + 2, kl - 1),      \
                                 Nout, a_base, b_base, acc, fa, fb);                            \
  } while (0)
  if (pw == 0) {
    gemm_issue(S0, a_rs, b_rs, Ld, wl, kb, Nout);
    gemm_issue(S1, a_rs, b_rs, Ld, wl, kb + min(1, kl - 1), Nout);
    asm volatile("s_waitcnt vmcnt(16) lgkmcnt(0)\n\ts_barrier" ::: "memory");   // step 0 landed
    switch (nv) {
      case 4: MOE_KLOOP(4, true, true); break;
      case 3: MOE_KLOOP(3, true, true); break;
      case 2: MOE_KLOOP(2, true, true); break;
      case 1: MOE_KLOOP(1, true, true); break;
      default: MOE_KLOOP(0, true, true); break;
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);          // vmcnt(0): no LDS write in flight at exit
  } else {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    switch (nv) {
      case 4: MOE_KLOOP(4, false, false); break;
      case 3: MOE_KLOOP(3, false, false); break;
      case 2: MOE_KLOOP(2, false, false); break;
      case 1: MOE_KLOOP(1, false, false); break;
      default: MOE_KLOOP(0, false, false); break;
    }
  }
#undef MOE_KLOOP

  // ---- k-range blocks: store the partial tile, and the last of a tile's
  // blocks to arrive sums all of its partials in range order (the order, and
  // so the result, does not depend on which block arrives last)
  if (!UP && slot >= 0) {
    // partial tiles through buffer instructions: the element offset goes in
    // the scalar offset, so no per-element address register is needed.  (Each
    // vector element is copied to a float before the bit cast: a bit cast of
    // the element expression itself compiled to element 0.)
    const __amdgpu_buffer_rsrc_t mine = __builtin_amdgcn_make_buffer_rsrc(
        part + (size_t)slot * (kBM * kBN), 0, kBM * kBN * 4, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = acc[i][j][r];
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), mine, tid * 4,
                                                ((i * 4 + j) * 4 + r) * kGemmThreads * 4, 0);
        }
    // every wave's stores are done before the barrier; one wave then makes the
    // block's tile visible device-wide (a release per block, not per wave:
    // each one writes back the XCD's L2)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int tile_sk = slot / segs;
    if (tid == 0) {
      __threadfence();
      const int last = atomicAdd(&tickets[tile_sk], 1) == segs - 1;
      if (last) __threadfence();       // acquire the other blocks' partial tiles
      s_last = last;
    }
    __syncthreads();
    if (!s_last) return;
    const __amdgpu_buffer_rsrc_t all = __builtin_amdgcn_make_buffer_rsrc(
        part + (size_t)tile_sk * segs * (kBM * kBN), 0, segs * kBM * kBN * 4, kRsrcWord3);
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
                                                            qo + ((i * 4 + j) * 4 + r) * kGemmThreads * 4, 0));
            acc[i][j][r] = q == 0 ? v : acc[i][j][r] + v;
          }
    }
  }

  // ---- epilogue: block (ib, jb), lane l, element r is row
  // 64 (ib >> 1) + 32 wm + 16 (ib & 1) + 4 (l >> 4) + r, column 16 (jb & 1) + (l & 15)
  // of the wave's column group jb >> 1
  if (UP && h13) {
    // training: the tile's act and both projections ([h1 | h3] per row of h13) leave
    // through LDS so that they are written as 256-byte row pieces by 16-byte stores
    // (three 2-byte stores per element straight from the accumulators cost about a
    // tenth of the kernel).  Two passes of 128 tile rows; a row holds
    // [act 128 | h1 128 | h3 128] bf16 and 16 bytes of padding (784 bytes: the four
    // row groups of a write, 4 rows apart, start 16 banks apart); rows 0..63 in S0,
    // 64..127 in S1.
    constexpr int kRowE = 392;
    uint16_t* act = static_cast<uint16_t*>(out);
    const int g4 = 4 * (lane >> 4), l16 = lane & 15;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      // before the first pass the k-loop's last refills must have landed; before
      // the second only the LDS reads of the first pass's stores (the stores
      // themselves stay in flight)
      if (pass == 0)
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      else
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
      for (int ib = 4 * pass; ib < 4 * pass + 4; ++ib)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int lr = 64 * (ib >> 1) + 32 * wm + 16 * (ib & 1) + g4 + r - 128 * pass;
          uint16_t* lrow = (lr < 64 ? S0 : S1) + (lr & 63) * kRowE;
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int c = wn * 64 + 32 * pw + 16 * jj + l16;
            const float h1 = acc[ib][jj][r], h3 = acc[ib][2 + jj][r];
            const float gv = h1 * __builtin_amdgcn_rcpf(1.f + __expf(-h1)) * h3;
            lrow[c] = f32_to_bf16(gv);
            lrow[128 + c] = f32_to_bf16(h1);
            lrow[256 + c] = f32_to_bf16(h3);
          }
        }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      // wave w writes rows 16 w .. 16 w + 15 of the pass: 48 (row, piece) pairs, four
      // per instruction (16 lanes x 16 bytes each)
      uint4 pv[12];       // every piece is read before the first store is issued
#pragma unroll
      for (int i = 0; i < 12; ++i) {
        const int idx = 4 * i + (lane >> 4);
        const int prow = 16 * w + idx / 3, seg = idx % 3;
        const uint16_t* lrow = (prow < 64 ? S0 : S1) + (prow & 63) * kRowE;
        pv[i] = *reinterpret_cast<const uint4*>(lrow + 128 * seg + 8 * l16);
      }
#pragma unroll
      for (int i = 0; i < 12; ++i) {
        const int idx = 4 * i + (lane >> 4);
        const int prow = 16 * w + idx / 3, seg = idx % 3;
        const int row = r0 + 128 * pass + prow;
        const uint4 v = pv[i];
        if (row < rend) {
          uint16_t* dst = seg == 0 ? act + (size_t)row * Nout + n0
                                   : h13 + (size_t)row * 2 * Nout + (seg == 2 ? Nout : 0) + n0;
          *reinterpret_cast<uint4*>(dst + 8 * l16) = v;
        }
      }
    }
  } else if (UP) {
    uint16_t* act = static_cast<uint16_t*>(out);
#pragma unroll
    for (int ib = 0; ib < 8; ++ib)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = r0 + 64 * (ib >> 1) + 32 * wm + 16 * (ib & 1) + 4 * (lane >> 4) + r;
        if (row < rend) {
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const float h1 = acc[ib][jj][r], h3 = acc[ib][2 + jj][r];
            const float gv = h1 * __builtin_amdgcn_rcpf(1.f + __expf(-h1)) * h3;
            act[(size_t)row * Nout + n0 + wn * 64 + 32 * pw + 16 * jj + (lane & 15)] = f32_to_bf16(gv);
          }
        }
      }
  } else {
    // buffer stores over the tile's rows: rows past the tile's end fall outside
    // the resource's range and are dropped
    const __amdgpu_buffer_rsrc_t y_rs = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<float*>(out) + (size_t)r0 * Nout, 0, tile_rows * Nout * 4, kRsrcWord3);
    const int vbase = ((32 * wm + 4 * (lane >> 4)) * Nout + n0 + wn * 128 + 64 * pw + (lane & 15)) * 4;
#pragma unroll
    for (int ib = 0; ib < 8; ++ib)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int vo = vbase + (64 * (ib >> 1) + 16 * (ib & 1) + r) * Nout * 4;
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
          const float v = acc[ib][jb][r];
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), y_rs,
                                                vo + (32 * (jb >> 1) + 16 * (jb & 1)) * 4, 0, 0);
        }
      }
  }
}

// ---------------------------------------------------------------- few rows per expert
// Decode-shaped batches give each expert only a handful of rows, so the work
// is reading every active expert's weights once (HBM-bound).  A wave owns one
// (expert, group of rows, column slice): it streams its weight columns
// straight from global memory into registers and never touches LDS.  How
// many contiguous bytes of a weight row one load instruction covers decides
// the DRAM efficiency on this part (a plain streaming read measured 5.9, 6.6
// and 7.0 TB/s for 128-, 256- and 512-byte pieces per row), so the main
// variant below reads 512 contiguous bytes per row per instruction.
//
// Column-permuted B operand: a lane loads 8 k-rows of 8 adjacent weight
// columns (one 16-byte vector per row) and transposes the 8x8 block in
// registers, giving 8 MFMA B operands (8 consecutive k each); MFMA number c
// then produces, in the lane's output column, weight column base + c.
//
// grouped_gemm_bf16_rows_kernel (up to 64 rows, 16x16x32 MFMAs): lane
// l = 16g + j loads k-rows k0+8g .. +7; for `up` lanes j < 8 read W1 columns
// n0 + 8j .. +7 and lanes j >= 8 the same columns of W3 (a shuffle across 8
// lanes pairs the SwiGLU halves); for `down` lane j reads W2 columns
// n0 + 8j .. +7 (128 columns).
template <bool UP, int MT>
__global__ __launch_bounds__(64) void grouped_gemm_bf16_rows_kernel(
    const uint16_t* __restrict__ X, const int32_t* __restrict__ offsets, int N,
    const uint16_t* __restrict__ Wa, const uint16_t* __restrict__ Wb, int K, int Nout,
    int n_slices, int max_rows, void* __restrict__ out) {
  constexpr int BM = 16 * MT;
  const int mt = blockIdx.x / n_slices, ns = blockIdx.x - mt * n_slices;
  int e, r0, rend;
  if (!find_tile(offsets, N, mt, BM, max_rows, e, r0, rend)) return;
  e = __builtin_amdgcn_readfirstlane(e);
  r0 = __builtin_amdgcn_readfirstlane(r0);
  rend = __builtin_amdgcn_readfirstlane(rend);

  const int lane = threadIdx.x, j = lane & 15, g = lane >> 4;
  const int n0 = ns * (UP ? 64 : 128);
  const size_t wexp = (size_t)e * K * Nout;
  const uint16_t* wsrc = UP ? ((j < 8 ? Wa : Wb) + wexp + n0 + 8 * (j & 7))
                            : (Wa + wexp + n0 + 8 * j);
  wsrc += (size_t)(8 * g) * Nout;
  // A rows: row r0 + 16 t + j (clamped to the last valid row), k 8g .. 8g+7
  const uint16_t* asrc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int row = min(r0 + 16 * t + j, rend - 1);
    asrc[t] = X + (size_t)row * K + 8 * g;
  }

  f32x4 acc[MT][8];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  const size_t rstride = (size_t)Nout;
  uint4 wb[2][8], xa[2][MT];
#define MOE_ROWS_LOAD(S, k0)                                                          \
  do {                                                                               \
    _Pragma("unroll") for (int kk = 0; kk < 8; ++kk)                                 \
        wb[S][kk] = load_stream(wsrc + (size_t)((k0) + kk) * rstride);               \
    _Pragma("unroll") for (int t = 0; t < MT; ++t)                                   \
        xa[S][t] = *reinterpret_cast<const uint4*>(asrc[t] + (k0));                  \
  } while (0)
#define MOE_ROWS_MMA(S)                                                               \
  do {                                                                               \
    uint4 bf[8];                                                                     \
    transpose8x8(wb[S], bf);                                                         \
    _Pragma("unroll") for (int t = 0; t < MT; ++t)                                   \
        _Pragma("unroll") for (int c = 0; c < 8; ++c)                                \
            acc[t][c] = mfma16(xa[S][t], bf[c], acc[t][c]);                          \
  } while (0)

  const int nk = K / 32;                        // K is a multiple of 64: nk is even
  MOE_ROWS_LOAD(0, 0);
  for (int kt = 0; kt < nk; kt += 2) {
    MOE_ROWS_LOAD(1, (kt + 1) * 32);
    MOE_ROWS_MMA(0);
    if (kt + 2 < nk) MOE_ROWS_LOAD(0, (kt + 2) * 32);
    MOE_ROWS_MMA(1);
  }
#undef MOE_ROWS_LOAD
#undef MOE_ROWS_MMA

  // acc[t][c][r]: row r0 + 16t + 4g + r, weight column base(j) + c
  if (UP) {
    uint16_t* act = static_cast<uint16_t*>(out);
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const float mine = acc[t][c][r];
          const float other = __shfl_xor(mine, 8, 64);    // W3 half for lanes j < 8
          v[c] = mine * __builtin_amdgcn_rcpf(1.f + __expf(-mine)) * other;
        }
        const int row = r0 + 16 * t + 4 * g + r;
        if (j < 8 && row < rend) {
          const uint4 pk = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                      pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
          *reinterpret_cast<uint4*>(act + (size_t)row * Nout + n0 + 8 * j) = pk;
        }
      }
  } else {
    float* y = static_cast<float*>(out);
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = r0 + 16 * t + 4 * g + r;
        if (row < rend) {
          float4* dst = reinterpret_cast<float4*>(y + (size_t)row * Nout + n0 + 8 * j);
          dst[0] = make_float4(acc[t][0][r], acc[t][1][r], acc[t][2][r], acc[t][3][r]);
          dst[1] = make_float4(acc[t][4][r], acc[t][5][r], acc[t][6][r], acc[t][7][r]);
        }
      }
  }
}

// Weight streaming with 32x32x16 MFMAs: a wave owns (expert, 32 rows, 256
// weight columns of one k-row per instruction: 32 lanes x 16 bytes = 512
// contiguous bytes).  Lane 32h + i loads k-rows k0 + 8h .. +7 of columns
// 8i .. 8i+7 of its block and transposes them in registers; MFMA c then
// yields, in output column i, weight column 8i + c.  UP: lanes i < 16 read W1
// columns n0 + 8i .., lanes i >= 16 the same W3 columns (128 activation
// columns per wave; a lane shuffle pairs the SwiGLU halves); DOWN: 256
// columns of W2.
template <bool UP>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 8))) void grouped_gemm_bf16_rows32_kernel(
    const uint16_t* __restrict__ X, const int32_t* __restrict__ offsets, int N,
    const uint16_t* __restrict__ Wa, const uint16_t* __restrict__ Wb, int K, int Nout,
    int n_slices, int max_rows, void* __restrict__ out) {
  const int mt = blockIdx.x / n_slices, ns = blockIdx.x - mt * n_slices;
  int e, r0, rend;
  if (!find_tile(offsets, N, mt, 32, max_rows, e, r0, rend)) return;
  e = __builtin_amdgcn_readfirstlane(e);
  r0 = __builtin_amdgcn_readfirstlane(r0);
  rend = __builtin_amdgcn_readfirstlane(rend);

  const int lane = threadIdx.x, i = lane & 31, h = lane >> 5;
  const int n0 = ns * (UP ? 128 : 256);
  const size_t wexp = (size_t)e * K * Nout;
  const uint16_t* wsrc = UP ? ((i < 16 ? Wa : Wb) + wexp + n0 + 8 * (i & 15))
                            : (Wa + wexp + n0 + 8 * i);
  wsrc += (size_t)(8 * h) * Nout;
  const uint16_t* asrc = X + (size_t)min(r0 + i, rend - 1) * K + 8 * h;

  f32x16 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;

  const size_t rstride = (size_t)Nout;
  uint4 wb[2][8], xa[2];
#define MOE_R32_LOAD(S, k0)                                                           \
  do {                                                                               \
    _Pragma("unroll") for (int kk = 0; kk < 8; ++kk)                                 \
        wb[S][kk] = load_stream(wsrc + (size_t)((k0) + kk) * rstride);               \
    xa[S] = *reinterpret_cast<const uint4*>(asrc + (k0));                            \
  } while (0)
#define MOE_R32_MMA(S)                                                                \
  do {                                                                               \
    uint4 bf[8];                                                                     \
    transpose8x8(wb[S], bf);                                                         \
    _Pragma("unroll") for (int c = 0; c < 8; ++c) acc[c] = mfma32(xa[S], bf[c], acc[c]); \
  } while (0)

  const int nk = K / 16;                        // K is a multiple of 64: nk is even
  MOE_R32_LOAD(0, 0);
  for (int kt = 0; kt < nk; kt += 2) {
    MOE_R32_LOAD(1, (kt + 1) * 16);
    MOE_R32_MMA(0);
    if (kt + 2 < nk) MOE_R32_LOAD(0, (kt + 2) * 16);
    MOE_R32_MMA(1);
  }
#undef MOE_R32_LOAD
#undef MOE_R32_MMA

  // acc[c][r]: row r0 + 8 (r / 4) + 4h + r % 4, column (of lane i's block) 8i + c
  if (UP) {
    uint16_t* act = static_cast<uint16_t*>(out);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float v[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float mine = acc[c][r];
        const float other = __shfl_xor(mine, 16, 64);    // W3 half for lanes i < 16
        v[c] = mine * __builtin_amdgcn_rcpf(1.f + __expf(-mine)) * other;
      }
      const int row = r0 + 8 * (r >> 2) + 4 * h + (r & 3);
      if (i < 16 && row < rend) {
        const uint4 pk = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                    pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
        *reinterpret_cast<uint4*>(act + (size_t)row * Nout + n0 + 8 * i) = pk;
      }
    }
  } else {
    float* y = static_cast<float*>(out);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = r0 + 8 * (r >> 2) + 4 * h + (r & 3);
      if (row < rend) {
        float4* dst = reinterpret_cast<float4*>(y + (size_t)row * Nout + n0 + 8 * i);
        dst[0] = make_float4(acc[0][r], acc[1][r], acc[2][r], acc[3][r]);
        dst[1] = make_float4(acc[4][r], acc[5][r], acc[6][r], acc[7][r]);
      }
    }
  }
}

// Up projection with 512-byte weight pieces: a block of two waves owns
// (expert, 32 rows, 256 activation columns); wave 0 streams those columns of W1
// and wave 1 the same columns of W3, each exactly as the down projection
// streams W2 (32 lanes cover 512 contiguous bytes of a k-row).  The SwiGLU
// halves meet in LDS: wave 0 hands over its W1 sums of the upper 16
// accumulator rows, wave 1 its W3 sums of the lower 16, and each wave
// finishes and stores half of the rows.
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2, 8))) void grouped_gemm_bf16_rows32_up2_kernel(
    const uint16_t* __restrict__ X, const int32_t* __restrict__ offsets, int N,
    const uint16_t* __restrict__ W1, const uint16_t* __restrict__ W3, int K, int F,
    int n_slices, int max_rows, uint16_t* __restrict__ act) {
  __shared__ float xch[2][8 * 8 * 64];      // [wave that wrote][c][half-row r][lane]
  const int mt = blockIdx.x / n_slices, ns = blockIdx.x - mt * n_slices;
  int e, r0, rend;
  if (!find_tile(offsets, N, mt, 32, max_rows, e, r0, rend)) return;
  e = __builtin_amdgcn_readfirstlane(e);
  r0 = __builtin_amdgcn_readfirstlane(r0);
  rend = __builtin_amdgcn_readfirstlane(rend);

  const int lane = threadIdx.x & 63, i = lane & 31, h = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int n0 = ns * 256;
  const uint16_t* wsrc = (w == 0 ? W1 : W3) + (size_t)e * K * F + n0 + 8 * i + (size_t)(8 * h) * F;
  const uint16_t* asrc = X + (size_t)min(r0 + i, rend - 1) * K + 8 * h;

  f32x16 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;

  const size_t rstride = (size_t)F;
  uint4 wb[2][8], xa[2];
#define MOE_U2_LOAD(S, k0)                                                            \
  do {                                                                               \
    _Pragma("unroll") for (int kk = 0; kk < 8; ++kk)                                 \
        wb[S][kk] = load_stream(wsrc + (size_t)((k0) + kk) * rstride);               \
    xa[S] = *reinterpret_cast<const uint4*>(asrc + (k0));                            \
  } while (0)
#define MOE_U2_MMA(S)                                                                 \
  do {                                                                               \
    uint4 bf[8];                                                                     \
    transpose8x8(wb[S], bf);                                                         \
    _Pragma("unroll") for (int c = 0; c < 8; ++c) acc[c] = mfma32(xa[S], bf[c], acc[c]); \
  } while (0)

  const int nk = K / 16;                        // K is a multiple of 64: nk is even
  MOE_U2_LOAD(0, 0);
  for (int kt = 0; kt < nk; kt += 2) {
    MOE_U2_LOAD(1, (kt + 1) * 16);
    MOE_U2_MMA(0);
    if (kt + 2 < nk) MOE_U2_LOAD(0, (kt + 2) * 16);
    MOE_U2_MMA(1);
  }
#undef MOE_U2_LOAD
#undef MOE_U2_MMA

  // acc[c][r]: row r0 + 8 (r / 4) + 4h + r % 4, column n0 + 8i + c.  Wave 0
  // keeps r < 8 and hands over r >= 8; wave 1 the other way round.
  const int keep = (w == 0) ? 0 : 8;
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const float v = (w == 0) ? acc[c][8 + rr] : acc[c][rr];
      xch[w][(c * 8 + rr) * 64 + lane] = v;
    }
  __syncthreads();
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) {
    float v[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float mine = (w == 0) ? acc[c][rr] : acc[c][8 + rr];
      const float other = xch[1 - w][(c * 8 + rr) * 64 + lane];
      const float g1 = (w == 0) ? mine : other, g3 = (w == 0) ? other : mine;
      v[c] = g1 * __builtin_amdgcn_rcpf(1.f + __expf(-g1)) * g3;
    }
    const int r = keep + rr;
    const int row = r0 + 8 * (r >> 2) + 4 * h + (r & 3);
    if (row < rend) {
      const uint4 pk = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                  pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
      *reinterpret_cast<uint4*>(act + (size_t)row * F + n0 + 8 * i) = pk;
    }
  }
}

template <bool UP>
static void launch_rows32(const void* x, const int32_t* offsets, int N, const void* wa,
                          const void* wb, int K, int Nout, int max_rows, void* out,
                          hipStream_t stream) {
  const int m_bound = (max_rows + 31) / 32 + N;
  if (UP && Nout % 256 == 0) {
    const int n_slices = Nout / 256;
    hipLaunchKernelGGL(grouped_gemm_bf16_rows32_up2_kernel, dim3(m_bound * n_slices), dim3(128), 0,
                       stream, static_cast<const uint16_t*>(x), offsets, N,
                       static_cast<const uint16_t*>(wa), static_cast<const uint16_t*>(wb), K, Nout,
                       n_slices, max_rows, static_cast<uint16_t*>(out));
    return;
  }
  const int n_slices = Nout / (UP ? 128 : 256);
  hipLaunchKernelGGL((grouped_gemm_bf16_rows32_kernel<UP>), dim3(m_bound * n_slices), dim3(64), 0,
                     stream, static_cast<const uint16_t*>(x), offsets, N,
                     static_cast<const uint16_t*>(wa), static_cast<const uint16_t*>(wb), K, Nout,
                     n_slices, max_rows, out);
}

// Few rows per expert: 0 = the MFMA tile kernel; 1 = 32-row weight streaming
// (average <= 32 rows per expert); 4 = 64-row weight streaming (<= 48).
static int rows_mt(int max_rows, int N) {
  const int avg = (max_rows + N - 1) / N;
  if (avg > 48) return 0;
  return avg <= 32 ? 1 : 4;
}

template <bool UP>
static void launch_rows(int mt, const void* x, const int32_t* offsets, int N, const void* wa,
                        const void* wb, int K, int Nout, int max_rows, void* out,
                        hipStream_t stream) {
  if (mt == 1) {
    launch_rows32<UP>(x, offsets, N, wa, wb, K, Nout, max_rows, out, stream);
    return;
  }
  const int n_slices = Nout / (UP ? 64 : 128);
  const int m_bound = (max_rows + 63) / 64 + N;
  hipLaunchKernelGGL((grouped_gemm_bf16_rows_kernel<UP, 4>), dim3(m_bound * n_slices), dim3(64), 0,
                     stream, static_cast<const uint16_t*>(x), offsets, N,
                     static_cast<const uint16_t*>(wa), static_cast<const uint16_t*>(wb), K, Nout,
                     n_slices, max_rows, out);
}

// ---------------------------------------------------------------- fp32 (VALU)
// 64-deep k chunks: each thread has BM / 4 loads of A and 16 (+16) of the weights
// in flight per chunk, so that a small layer (a few chunks per block) waits on
// memory a few times rather than K / 16 times.  The k order of every sum is
// unchanged.  Tiles of BM = 64 rows, or 16 when the experts average at most 16
// rows: the arithmetic of a 64-row tile runs on the waves that hold its rows,
// so a tile with 16 real rows would leave three of its four waves idle.
constexpr int kFBN = 64, kFBK = 64;

template <bool UP, int BM>
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(
    const float* __restrict__ X, const int32_t* __restrict__ offsets, int N,
    const float* __restrict__ Wa, const float* __restrict__ Wb, int K, int Nout, int n_tiles,
    int max_rows, float* __restrict__ out, float* __restrict__ h13) {
  constexpr int RPT = BM / 16;                  // rows per thread
  __shared__ float As[kFBK][BM + 1];
  __shared__ float B1[kFBK][kFBN];
  __shared__ float B3[kFBK][kFBN];
  const int mt = blockIdx.x / n_tiles, nt = blockIdx.x % n_tiles;
  int e, r0, rend;
  if (!find_tile(offsets, N, mt, BM, max_rows, e, r0, rend)) return;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int n0 = nt * kFBN;
  const size_t wexp = (size_t)e * K * Nout;
  float c1[RPT][4] = {}, c3[RPT][4] = {};
  for (int k0 = 0; k0 < K; k0 += kFBK) {
    float va[BM / 4], vb1[16], vb3[16];
#pragma unroll
    for (int i = 0; i < BM / 4; ++i) {
      const int item = tid + 256 * i;           // BM rows x 64 k
      const int row = item >> 6, kk = item & 63;
      const int gr = r0 + row;
      va[i] = gr < rend ? X[(size_t)gr * K + k0 + kk] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int item = tid + 256 * i;
      const int kr = item >> 6, col = item & 63;  // 64 k x 64 cols
      vb1[i] = Wa[wexp + (size_t)(k0 + kr) * Nout + n0 + col];
      vb3[i] = UP ? Wb[wexp + (size_t)(k0 + kr) * Nout + n0 + col] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < BM / 4; ++i) {
      const int item = tid + 256 * i;
      As[item & 63][item >> 6] = va[i];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int item = tid + 256 * i;
      B1[item >> 6][item & 63] = vb1[i];
      if (UP) B3[item >> 6][item & 63] = vb3[i];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kFBK; ++kk) {
      float a[RPT], b1[4], b3[4];
#pragma unroll
      for (int i = 0; i < RPT; ++i) a[i] = As[kk][ty * RPT + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        b1[j] = B1[kk][tx * 4 + j];
        if (UP) b3[j] = B3[kk][tx * 4 + j];
      }
#pragma unroll
      for (int i = 0; i < RPT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          c1[i][j] = fmaf(a[i], b1[j], c1[i][j]);
          if (UP) c3[i][j] = fmaf(a[i], b3[j], c3[i][j]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = r0 + ty * RPT + i;
    if (row >= rend) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      float v = c1[i][j];
      if (UP && h13) {
        h13[(size_t)row * 2 * Nout + col] = v;
        h13[(size_t)row * 2 * Nout + Nout + col] = c3[i][j];
      }
      if (UP) v = v / (1.f + expf(-v)) * c3[i][j];
      out[(size_t)row * Nout + col] = v;
    }
  }
}

// Row tile of the fp32 kernel: 16 rows when the experts average at most 16.
static bool f32_small_tiles(int max_rows, int N) { return (max_rows + N - 1) / N <= 16; }

template <bool UP>
static void launch_f32(const float* x, const int32_t* offsets, int N, const float* wa,
                       const float* wb, int K, int Nout, int max_rows, float* out, float* h13,
                       hipStream_t stream) {
  const int n_tiles = Nout / kFBN;
  if (f32_small_tiles(max_rows, N)) {
    const int mt_bound = (max_rows + 15) / 16 + N;
    hipLaunchKernelGGL((grouped_gemm_f32_kernel<UP, 16>), dim3(mt_bound * n_tiles), dim3(256), 0,
                       stream, x, offsets, N, wa, wb, K, Nout, n_tiles, max_rows, out, h13);
  } else {
    const int mt_bound = (max_rows + 63) / 64 + N;
    hipLaunchKernelGGL((grouped_gemm_f32_kernel<UP, 64>), dim3(mt_bound * n_tiles), dim3(256), 0,
                       stream, x, offsets, N, wa, wb, K, Nout, n_tiles, max_rows, out, h13);
  }
}

static int round8(int x) { return (x + 7) & ~7; }

// Compute units of the current device (cached per device; calls from several
// host threads may query the same device concurrently, so the cache is atomic).
int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = cus[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cus[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

__global__ void zero_tickets_kernel(int32_t* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// Workspace of the down projection: one fp32 256 x 256 partial tile and one
// ticket per CU for the k-split last round (MFMA path only).
static size_t partial_bytes(int cus) { return (size_t)cus * kBM * kBN * sizeof(float); }

size_t expert_down_ws_bytes(int N, int d, int f, int max_rows, bool bf16) {
  (void)d;
  (void)f;
  if (!bf16 || rows_mt(max_rows, N) > 0) return 0;
  const int cus = device_cus();
  if (cus <= 0) return 0;
  return partial_bytes(cus) + (((size_t)cus * sizeof(int32_t) + 255) & ~(size_t)255);
}

hipError_t launch_expert_up(const void* x_perm, const int32_t* offsets, const void* w1,
                            const void* w3, int N, int d, int f, int max_rows, bool bf16,
                            void* act, void* h13, hipStream_t stream) {
  // with h13 (training) the tile kernels run at every batch size: only they store h1 / h3
  if (bf16 && !h13 && rows_mt(max_rows, N) > 0) {
    launch_rows<true>(rows_mt(max_rows, N), x_perm, offsets, N, w1, w3, d, f, max_rows, act, stream);
  } else if (bf16) {
    const int n_tiles = f / (kBN / 2);
    const int mt_bound = (max_rows + kBM - 1) / kBM + N;
    const int grid = round8(mt_bound * n_tiles);
    hipLaunchKernelGGL(grouped_gemm_bf16_kernel<true>, dim3(grid), dim3(kGemmThreads), 0, stream,
                       static_cast<const uint16_t*>(x_perm), offsets, N,
                       static_cast<const uint16_t*>(w1), static_cast<const uint16_t*>(w3), d, f,
                       n_tiles, max_rows, act, static_cast<float*>(nullptr),
                       static_cast<int32_t*>(nullptr), device_cus(), grid,
                       static_cast<uint16_t*>(h13));
  } else {
    launch_f32<true>(static_cast<const float*>(x_perm), offsets, N, static_cast<const float*>(w1),
                     static_cast<const float*>(w3), d, f, max_rows, static_cast<float*>(act),
                     static_cast<float*>(h13), stream);
  }
  return hipGetLastError();
}

hipError_t launch_expert_down(const void* act, const int32_t* offsets, const void* w2, int N,
                              int d, int f, int max_rows, bool bf16, float* y_perm, void* ws,
                              hipStream_t stream) {
  if (bf16 && rows_mt(max_rows, N) > 0) {
    launch_rows<false>(rows_mt(max_rows, N), act, offsets, N, w2, nullptr, f, d, max_rows,
                       static_cast<void*>(y_perm), stream);
  } else if (bf16) {
    const int n_tiles = d / kBN;
    const int mt_bound = (max_rows + kBM - 1) / kBM + N;
    const int dp_grid = round8(mt_bound * n_tiles);
    const int cus = device_cus();
    // the last round is split over k only for tiles of at least kMinSplitSteps
    // k-steps: for shallower ones the tickets are never used, so they are not
    // cleared and no range blocks are launched
    const bool may_split = f / kBK >= kMinSplitSteps;
    float* part = (cus > 0 && may_split) ? static_cast<float*>(ws) : nullptr;
    int32_t* tickets = nullptr;
    int grid = dp_grid;
    if (part) {
      tickets = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + partial_bytes(cus));
      hipLaunchKernelGGL(zero_tickets_kernel, dim3((cus + 255) / 256), dim3(256), 0, stream,
                         tickets, cus);
      grid += round8(cus);
    }
    hipLaunchKernelGGL(grouped_gemm_bf16_kernel<false>, dim3(grid), dim3(kGemmThreads), 0, stream,
                       static_cast<const uint16_t*>(act), offsets, N,
                       static_cast<const uint16_t*>(w2), static_cast<const uint16_t*>(nullptr), f,
                       d, n_tiles, max_rows, static_cast<void*>(y_perm), part, tickets, cus,
                       dp_grid, static_cast<uint16_t*>(nullptr));
  } else {
    launch_f32<false>(static_cast<const float*>(act), offsets, N, static_cast<const float*>(w2),
                      nullptr, f, d, max_rows, y_perm, nullptr, stream);
  }
  return hipGetLastError();
}

}  // namespace moe
