/*
 * moe.h -- C ABI of libmoe_mi355x.so: the forward pass of a top-k routed
 * Mixture-of-Experts SwiGLU FFN layer on one MI355X (gfx950).
 *
 * Pages cited (named by address; none has a usable title line):
 *   P1 cf-1.com/news/5914943            P2 hotelren.com/news/5904824
 *   P3 devpress.csdn.net/awstech/6a91abf42b83d06f0ec71b09.html
 *   P4 2kiu.com/news/2885792            P5 hotelren.com/news/3071227
 *
 * The layer (P1 §2.1, P1 §2.3, P4 §2.2, P4 §3.1):
 *   logits  = hidden . W_router (+ bias)                          moe_route
 *   top-k per token, softmax over the k selected logits           moe_route
 *   per-expert counts, capacity cut, expert-contiguous permute    moe_permute
 *   (or: over-capacity assignments re-routed once)                moe_permute_reroute
 *   per-expert SwiGLU FFN as one grouped GEMM pair                moe_expert_ffn
 *   weighted combine back to token order (+ shared experts)       moe_combine
 *   load-balancing loss N * sum_e f_e * P_e                       moe_aux_loss
 *
 * Its backward (gradients of <dy, y> + aux_coef * aux; P1 §2.3, P4 §2.2,
 * P4 §5.1):
 *   through the combine                                           moe_combine_backward
 *   through both grouped GEMMs (dx, dW1, dW3, dW2)               moe_expert_backward
 *   (or with h1, h3 kept by the forward's moe_expert_up_save)     moe_expert_backward_saved
 *   through the softmax, the aux loss and the router linear       moe_router_backward
 *
 * Conventions shared by every entry point:
 *   - Every pointer argument is a DEVICE pointer owned by the caller, to a
 *     contiguous row-major array, 16-byte aligned (the kernels use 16-byte
 *     accesses; hipMalloc and torch allocations are 256-byte aligned; a
 *     misaligned pointer is MOE_ERR_INVALID_ARG); the library never
 *     allocates, frees, keeps or synchronises.  `stream` is a hipStream_t
 *     passed as void* (NULL = the null stream); all work is enqueued on it
 *     asynchronously.
 *   - Argument errors are detected on the host before anything is enqueued
 *     and leave every output untouched.  MOE_ERR_HIP reports a launch error;
 *     a fault inside a kernel surfaces at the caller's next synchronisation.
 *   - dtype MOE_BF16: hidden, weights, x_perm, the SwiGLU activations and y
 *     are bfloat16 (raw 16-bit patterns); accumulation is fp32.  MOE_F32: all
 *     of them are fp32.  logits, topk_w, y_perm and aux are always fp32.
 *   - Limits: 1 <= k <= N <= 256; T >= 1; d and f multiples of 64; for the
 *     bf16 expert GEMMs also d a multiple of 256 and f of 128 and d < 2^21
 *     (a 256-row fp32 tile of y_perm under 2^31 bytes); one expert matrix
 *     (d * f elements) under 2^31 bytes; T * k < 2^31.  Outside them:
 *     MOE_ERR_UNSUPPORTED.
 *   - Inputs must be finite; behaviour on NaN/Inf inputs is unspecified.
 *   - Calls on one stream are ordered; calls that share outputs or workspace
 *     on different streams race.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null or misaligned pointer, non-positive size, k outside [1, N], NaN capacity factor */
  MOE_ERR_UNSUPPORTED = 2, /* shape or dtype outside the limits above */
  MOE_ERR_WORKSPACE = 3,   /* workspace smaller than moe_workspace_size() */
  MOE_ERR_HIP = 4          /* HIP launch error */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef enum {
  MOE_OP_ROUTE = 0,
  MOE_OP_PERMUTE = 1,
  MOE_OP_EXPERT_FFN = 2,
  MOE_OP_COMBINE = 3,
  MOE_OP_AUX_LOSS = 4,
  MOE_OP_EXPERT_DOWN = 5,
  MOE_OP_PERMUTE_REROUTE = 6,
  MOE_OP_EXPERT_BACKWARD = 7,
  MOE_OP_ROUTER_BACKWARD = 8,
  MOE_OP_EXPERT_BACKWARD_SAVED = 9
} moe_op;

/* Human-readable name of a status code (static string). */
const char* moe_status_string(moe_status s);

/*
 * moe_capacity -- the per-expert capacity moe_permute and moe_permute_reroute
 * use (P4 §3.1: token slots T*k over N experts times the capacity factor,
 * truncated; P5 §2.2: 65536 tokens, 64 experts, factor 1.2 give 1228):
 *   C = floor(((double)T * k) / N * capacity_factor)   in IEEE double, in
 *   that operation order, for capacity_factor > 0; C = T when
 *   capacity_factor <= 0 (no limit) or when the formula reaches T or more
 *   (no expert can hold more than T rows: a token picks an expert at most
 *   once).  Host-only; touches no device.  Returns -1 for T < 1, N < 1,
 *   k < 1, k > N or a NaN capacity_factor.
 */
int moe_capacity(int T, int k, int N, double capacity_factor);

/* Bytes of device workspace `op` needs for these sizes (0 if none).  Returns
 * 0 for an unknown op as well.  For MOE_OP_EXPERT_FFN and MOE_OP_EXPERT_DOWN,
 * T*k is the row capacity (max_rows) of x_perm / y_perm.  The two expert ops
 * size their k-split buffers by the compute units of the CURRENT device
 * (0 when no device is visible); query with that device current.
 * MOE_OP_EXPERT_BACKWARD and MOE_OP_EXPERT_BACKWARD_SAVED: T*k is max_rows.
 * MOE_OP_ROUTER_BACKWARD: d and N of the router, T tokens. */
size_t moe_workspace_size(moe_op op, int T, int d, int N, int k, int f, moe_dtype dt);

/*
 * moe_route -- router linear layer, top-k, gate weights, pre-drop counts.
 *   P1 §2.1 (a small linear layer scores every expert, the top-k scores are
 *   kept and softmax-normalised), P4 §3.1 (logits = hidden . router_w with
 *   router_w [D, E]), P4 §5.3 (equal logits rank by ascending expert id),
 *   P1 §2.3 (tokens per expert).
 *
 *   hidden    [T, d]   dtype dt
 *   w_router  [d, N]   dtype dt
 *   bias      [N] fp32 per-expert logit offset, or NULL for none
 *   logits    [T, N] fp32 out: hidden . w_router (+ bias), fp32 accumulation
 *   topk_idx  [T, k] int32 out: expert ids ordered by (logit desc, id asc)
 *   topk_w    [T, k] fp32 out: softmax over the k selected logits
 *   counts    [N] int32 out: number of tokens that chose each expert (before
 *             any capacity drop); sum(counts) = T*k
 *   ws        device workspace of moe_workspace_size(MOE_OP_ROUTE, ...) bytes
 *             (bf16: w_router transposed when T >= 2048, else partial logits
 *             when the hidden dimension is split across blocks; may be NULL
 *             when that size is 0)
 */
moe_status moe_route(const void* hidden, const void* w_router, const float* bias, int T, int d,
                     int N, int k, moe_dtype dt, float* logits, int32_t* topk_idx, float* topk_w,
                     int32_t* counts, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_permute -- capacity cut and permutation into expert-contiguous rows.
 *   P4 §3.1 (the capacity is the token-slot count T*k shared evenly over the
 *   experts and scaled by the capacity factor, truncated to an integer; each
 *   expert keeps its first `capacity` tokens), P5 §2.2 (worked capacity
 *   example), P1 §2.3 tip (tokens over capacity skip the MoE FFN and ride the
 *   residual), P3 §4.1 (scatter tokens into per-expert queues instead of a
 *   per-expert loop).
 *
 *   capacity_factor > 0: C = moe_capacity(T, k, N, capacity_factor); <= 0:
 *   no limit (C = T).  Tokens take places at an expert in token order; (t, j)
 *   is kept iff its place is < C.  Kept rows are expert-major,
 *   token-ascending within an expert.
 *
 *   hidden    [T, d] dtype dt
 *   topk_idx  [T, k] int32 (from moe_route; ids outside [0, N) are ignored)
 *   x_perm    [T*k, d] dtype dt out: rows [0, offsets[N]) = gathered hidden
 *             rows (the rest are not written)
 *   perm_src  [T*k] int32 out: token of each kept row (rows >= offsets[N] not written)
 *   slot_row  [T, k] int32 out: row in x_perm of (t, j), or -1 if dropped
 *   kept      [N] int32 out: min(count_e, C)
 *   offsets   [N+1] int32 out: exclusive prefix sum of kept; offsets[N] = rows used
 *   ws        device workspace of moe_workspace_size(MOE_OP_PERMUTE, ...) bytes
 */
moe_status moe_permute(const void* hidden, const int32_t* topk_idx, int T, int d, int N, int k,
                       double capacity_factor, moe_dtype dt, void* x_perm, int32_t* perm_src,
                       int32_t* slot_row, int32_t* kept, int32_t* offsets, void* ws,
                       size_t ws_bytes, void* stream);

/*
 * moe_permute_noalloc -- moe_permute without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Same arguments, outputs,
 * results and errors as moe_permute, bit for bit; the chunk tables moe_permute
 * keeps in `ws` live instead in a static device array inside the library,
 * MOE_PERMUTE_NOALLOC_SCRATCH_BYTES (4 MiB) on each device it runs on, held
 * from the library's load until the process ends.  It allocates nothing,
 * frees nothing and synchronises nothing (its first call on a device looks
 * up that device's address of the array, host-side only).
 *   Limit: moe_workspace_size(MOE_OP_PERMUTE, T, ...) = 8 * ceil(T / 256) * N
 *   bytes must not exceed MOE_PERMUTE_NOALLOC_SCRATCH_BYTES (T * N <= 2^27
 *   or so, e.g. 524288 tokens at 256 experts), else MOE_ERR_WORKSPACE before
 *   anything is enqueued.
 *   Every call on one device uses that device's one array: calls that overlap
 *   on a device (different streams, or threads without ordering) race and
 *   give wrong results.  Order them, e.g. on one stream.  Nothing in the
 *   array needs to start at zero.
 */
#define MOE_PERMUTE_NOALLOC_SCRATCH_BYTES (4u << 20)
moe_status moe_permute_noalloc(const void* hidden, const int32_t* topk_idx, int T, int d, int N,
                               int k, double capacity_factor, moe_dtype dt, void* x_perm,
                               int32_t* perm_src, int32_t* slot_row, int32_t* kept,
                               int32_t* offsets, void* stream);

/*
 * moe_permute_reroute -- as moe_permute, but assignments over capacity get
 * one second chance instead of being dropped.  P5 §4.2 (capacity-aware
 * routing: mask the over-capacity pick, take the next-best expert), P4 §2.2
 * and P5 §2.2 (over-capacity tokens are dropped or sent to the next-best
 * expert), P3 §2.3 (overflow handed to idle experts).
 *
 *   First round exactly as moe_permute (kept1_e = min(count_e, C)).  Second
 *   round: each dropped (t, j), in slot order within token t, proposes the
 *   expert with the largest logits[t, e] (fp32; ties to the lower id) among
 *   experts that are not in topk_idx[t, :], were not proposed by an earlier
 *   dropped slot of t, and have kept1_e < C.  Each expert admits proposals in
 *   token order while it has room (C - kept1_e); the rest stay dropped.
 *   Inside an expert, first-round rows come first, then second-round rows,
 *   each token-ascending.  A moved slot keeps its gate weight: moe_combine
 *   needs no change.
 *
 *   logits  [T, N] fp32 (from moe_route)
 *   other arguments, outputs and limits as moe_permute; kept[e] counts both
 *   rounds (<= C)
 *   ws      moe_workspace_size(MOE_OP_PERMUTE_REROUTE, T, d, N, k, f, dt) bytes
 */
moe_status moe_permute_reroute(const void* hidden, const int32_t* topk_idx, const float* logits,
                               int T, int d, int N, int k, double capacity_factor, moe_dtype dt,
                               void* x_perm, int32_t* perm_src, int32_t* slot_row, int32_t* kept,
                               int32_t* offsets, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_expert_ffn -- every expert's SwiGLU FFN over its rows, as two grouped
 * GEMMs (P1 §3.3 grouped GEMM; P4 §3.3 one kernel for all experts indexed by
 * expert id; P4 §5.4 all experts' weights in one tensor sliced by id; P4 §2.2
 * SwiGLU experts):  y_perm[r] = (silu(x_perm[r] W1_e) * (x_perm[r] W3_e)) W2_e
 * for every row r in [offsets[e], offsets[e+1]), silu(z) = z / (1 + e^-z).
 * Equivalent to moe_expert_up followed by moe_expert_down with the
 * activations held in `ws`.
 *
 *   x_perm    [max_rows, d] dtype dt
 *   offsets   [N+1] int32 (from moe_permute; offsets[N] <= max_rows)
 *   w1, w3    [N, d, f] dtype dt;  w2 [N, f, d] dtype dt
 *   y_perm    [max_rows, d] fp32 out (rows >= offsets[N] not written)
 *   ws        moe_workspace_size(MOE_OP_EXPERT_FFN, T, d, N, k, f, dt) bytes
 *             with T*k = max_rows: the activations [max_rows, f] (padded to
 *             256 bytes), then moe_expert_down's workspace
 */
moe_status moe_expert_ffn(const void* x_perm, const int32_t* offsets, const void* w1,
                          const void* w3, const void* w2, int N, int d, int f, int max_rows,
                          moe_dtype dt, float* y_perm, void* ws, size_t ws_bytes, void* stream);

/* First grouped GEMM with the SwiGLU epilogue fused:
 *   act[r] = silu(x_perm[r] W1_e) * (x_perm[r] W3_e), act [max_rows, f] dtype dt. */
moe_status moe_expert_up(const void* x_perm, const int32_t* offsets, const void* w1,
                         const void* w3, int N, int d, int f, int max_rows, moe_dtype dt,
                         void* act, void* stream);

/* moe_expert_up for training: the same act, and also both projections
 *   h13[r, 0:f] = x_perm[r] W1_e,  h13[r, f:2f] = x_perm[r] W3_e
 * in dtype dt (bf16: rounded to nearest even), h13 [max_rows, 2f], for
 * moe_expert_backward_saved, which then needs no recompute of them.  Runs the
 * MFMA tile kernels at every batch size (they alone store h13).  Rows >=
 * offsets[N] of h13 are not written. */
moe_status moe_expert_up_save(const void* x_perm, const int32_t* offsets, const void* w1,
                              const void* w3, int N, int d, int f, int max_rows, moe_dtype dt,
                              void* act, void* h13, void* stream);

/* Second grouped GEMM: y_perm[r] = act[r] W2_e, y_perm fp32.
 *   ws  moe_workspace_size(MOE_OP_EXPERT_DOWN, T, d, N, k, f, dt) bytes with
 *       T*k = max_rows (may be NULL when that size is 0).  When the tiles'
 *       last round would leave most compute units idle, its tiles are split
 *       over k and the partial tiles meet in `ws`; they are summed in a fixed
 *       order, so results do not depend on scheduling.  Calls that share `ws`
 *       must be ordered (same stream). */
moe_status moe_expert_down(const void* act, const int32_t* offsets, const void* w2, int N, int d,
                           int f, int max_rows, moe_dtype dt, float* y_perm, void* ws,
                           size_t ws_bytes, void* stream);

/*
 * FP8 expert weights (P1 §3.1: experts stored in FP8) for decode-shaped
 * batches, where the layer's time is reading the active experts' weights
 * (P5 §2.2-2.3).  Format: OCP FP8 E4M3 (bias 7, 3 mantissa bits, subnormals,
 * largest finite 448, no infinity), one fp32 scale per output column of each
 * expert matrix.
 *
 * moe_quantize_fp8 -- per-column quantisation of N matrices w [N, K, M]
 *   (dtype dt; K = the reduction dimension): for every (e, m)
 *   scale[e, m] = max_k |w[e, k, m]| / 448 (1 if the column is all zero) and
 *   q[e, k, m] = round-to-nearest-even(w[e, k, m] / scale[e, m]) clamped to
 *   +-448, both divisions IEEE float32.  W1/W3 [N, d, f] give scales [N, f];
 *   W2 [N, f, d] gives scales [N, d].
 *   q [N, K, M] uint8 out, scale [N, M] fp32 out.
 */
moe_status moe_quantize_fp8(const void* w, moe_dtype dt, int N, int K, int M, uint8_t* q,
                            float* scale, void* stream);

/* moe_expert_up_fp8 / moe_expert_down_fp8 -- as moe_expert_up / moe_expert_down
 * (bf16 activations) with W = code * column scale:
 *   act[r] = silu((x_perm[r] Q1_e) * s1_e) * ((x_perm[r] Q3_e) * s3_e)
 *   y_perm[r] = (act[r] Q2_e) * s2_e
 * w1q, w3q [N, d, f] and w2q [N, f, d] uint8 codes, s1, s3 [N, f] and
 * s2 [N, d] fp32 (from moe_quantize_fp8).  They run on the weight-streaming
 * kernels only: the bf16 shape limits and ceil(max_rows / N) <= 32, else
 * MOE_ERR_UNSUPPORTED. */
moe_status moe_expert_up_fp8(const void* x_perm, const int32_t* offsets, const uint8_t* w1q,
                             const uint8_t* w3q, const float* s1, const float* s3, int N, int d,
                             int f, int max_rows, void* act, void* stream);
moe_status moe_expert_down_fp8(const void* act, const int32_t* offsets, const uint8_t* w2q,
                               const float* s2, int N, int d, int f, int max_rows, float* y_perm,
                               void* stream);

/*
 * moe_combine -- weighted combine back to token order (P1 §2.1: the output
 * is the gate-weighted sum of the selected experts' outputs; P3 §4.1 gather),
 * plus the shared experts (P2 §3.3: experts every token calls, added with
 * weight 1).
 *   y[t] = sum over j = 0..k-1 with slot_row[t, j] >= 0 of
 *          topk_w[t, j] * y_perm[slot_row[t, j]]
 *        + sum over q = 0..n_shared-1 of y_shared[q][t]
 *   summed in that order in fp32, then stored in dtype dt.  Dropped slots
 *   contribute nothing (weights are not renormalised); the residual is NOT
 *   added (the caller adds hidden + y).
 *   y_shared  [n_shared, T, d] fp32, the shared experts' FFN outputs (each one
 *             moe_expert_ffn over all T rows of hidden with offsets {0, T}),
 *             or NULL with n_shared = 0
 */
moe_status moe_combine(const float* y_perm, const int32_t* slot_row, const float* topk_w,
                       const float* y_shared, int n_shared, int T, int d, int k, moe_dtype dt,
                       void* y, void* stream);

/*
 * moe_aux_loss -- load-balancing loss (P1 §2.3; P2 §3.2):
 *   aux = N * sum_e f_e * P_e,  f_e = counts[e] / (T*k)  (pre-drop),
 *   P_e = (1/T) sum_t softmax(logits[t, :])_e  (softmax over all N).
 *   Equals 1 when routing is uniform.  The caller applies its coefficient.
 *
 *   logits [T, N] fp32, counts [N] int32 (from moe_route), aux: 1 fp32 out.
 */
moe_status moe_aux_loss(const float* logits, const int32_t* counts, int T, int N, int k,
                        float* aux, void* ws, size_t ws_bytes, void* stream);

/*
 * Backward pass.  The top-k choice, the capacity cut and the counts are
 * piecewise constant and pass no gradient; gradients reach the router through
 * the softmax over the k selected logits and through P_e of the aux loss
 * (P4 §5.1: only the selected experts get a gradient).  Every gradient output
 * is fp32.  Inputs are the forward's outputs for the same batch (moe_route,
 * moe_permute or moe_permute_reroute, moe_expert_ffn).
 *
 * moe_combine_backward -- for every kept slot (t, j), r = slot_row[t, j]:
 *   g_perm[r]   = topk_w[t, j] * dy[t]            (dtype dt)
 *   dgate[t, j] = <dy[t], y_perm[r]>              (fp32; 0 for dropped slots)
 *   dy [T, d] dtype dt; y_perm [max_rows, d] fp32 (moe_expert_ffn);
 *   g_perm [max_rows, d] dtype dt out (rows >= offsets[N] not written);
 *   dgate [T, k] fp32 out.
 */
moe_status moe_combine_backward(const void* dy, const float* y_perm, const int32_t* slot_row,
                                const float* topk_w, int T, int d, int k, moe_dtype dt,
                                void* g_perm, float* dgate, void* stream);

/*
 * moe_expert_backward -- backward of every expert's SwiGLU FFN (P4 §2.2: each
 * expert has gradients of its own), for rows r of expert e (h1 = x_perm[r] W1_e,
 * h3 = x_perm[r] W3_e recomputed, s = sigmoid(h1), a = h1 s h3,
 * da = g_perm[r] W2_e^T, dh1 = da h3 (s + h1 s (1 - s)), dh3 = da h1 s):
 *   dx_perm[r] = dh1 W1_e^T + dh3 W3_e^T           [max_rows, d] fp32 out
 *   dw1[e] = sum_r x_perm[r]^T dh1,  dw3[e] = sum_r x_perm[r]^T dh3     [N, d, f] fp32 out
 *   dw2[e] = sum_r a^T g_perm[r]                                        [N, f, d] fp32 out
 * An expert with no rows gets zero weight gradients.  Rows >= offsets[N] of
 * dx_perm are not written.
 *   x_perm, g_perm [max_rows, d] dtype dt; offsets [N+1]; w1, w3 [N, d, f],
 *   w2 [N, f, d] dtype dt.
 *   ws  moe_workspace_size(MOE_OP_EXPERT_BACKWARD, T, d, N, k, f, dt) bytes,
 *       T*k = max_rows: da [max_rows, f] fp32, [dh1 | dh3] [max_rows, 2f] and
 *       a [max_rows, f] in dtype dt, each padded to 256 bytes, and for bf16
 *       one fp32 256 x 256 tile and one counter per compute unit of the
 *       current device: when the dx GEMM's last round of tiles would leave
 *       most compute units idle, those tiles are split over k and their
 *       partial tiles meet there, summed in a fixed order (results do not
 *       depend on scheduling).  Calls that share `ws` must be ordered.
 *   Limits: those of moe_expert_ffn; for bf16 f a multiple of 256,
 *   max_rows * f < 2^29 and max_rows * d < 2^30.
 */
moe_status moe_expert_backward(const void* x_perm, const void* g_perm, const int32_t* offsets,
                               const void* w1, const void* w3, const void* w2, int N, int d,
                               int f, int max_rows, moe_dtype dt, float* dx_perm, float* dw1,
                               float* dw3, float* dw2, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_expert_backward_saved -- moe_expert_backward with h1 and h3 taken from
 * the h13 [max_rows, 2f] that moe_expert_up_save stored in the forward
 * (dtype dt) instead of recomputed from x_perm: the SwiGLU backward (dh1,
 * dh3) runs in the epilogue of the da GEMM, so the backward does 12 A d f
 * flops instead of 16 (no recompute GEMM).
 *   act  NULL, or the forward's activations [max_rows, f] (dtype dt; the
 *        `act` moe_expert_up_save wrote): dW2 = act^T g then uses the very
 *        values the forward multiplied by W2, and the epilogue neither
 *        recomputes nor writes a.  With NULL, a = silu(h1) h3 is recomputed
 *        from h13 into the workspace.
 * Arguments, outputs and limits otherwise as moe_expert_backward.
 *   ws  moe_workspace_size(MOE_OP_EXPERT_BACKWARD_SAVED, T, d, N, k, f, dt)
 *       bytes, T*k = max_rows: [dh1 | dh3] [max_rows, 2f] and a [max_rows, f]
 *       in dtype dt, each padded to 256 bytes, and (bf16) the dx GEMM's k-split
 *       tiles and counters as for moe_expert_backward.
 */
moe_status moe_expert_backward_saved(const void* x_perm, const void* g_perm, const void* h13,
                                     const void* act, const int32_t* offsets, const void* w1,
                                     const void* w3, const void* w2, int N, int d, int f,
                                     int max_rows, moe_dtype dt, float* dx_perm, float* dw1,
                                     float* dw3, float* dw2, void* ws, size_t ws_bytes,
                                     void* stream);

/*
 * moe_router_backward -- through the softmax over the k selected logits, the
 * aux loss (coefficient aux_coef, P1 §2.3) and the router linear:
 *   dlogit[t, e] = aux_coef (N / T) p[t, e] (f_e - sum_m p[t, m] f_m)
 *                  (p = softmax over all N, f_e = counts[e] / (T k))
 *                + sum_j [topk_idx[t, j] = e] topk_w[t, j] (dgate[t, j] - sum_m topk_w[t, m] dgate[t, m])
 *   dhidden[t]   = sum_j dx_perm[slot_row[t, j]] (kept slots) + dlogit[t] W_router^T
 *                  + sum_q dx_shared[q][t]
 *   dw_router    = hidden^T dlogit  [d, N] fp32 out
 *   dbias        = sum_t dlogit[t]  [N] fp32 out, or NULL to skip
 *   hidden [T, d], w_router [d, N] dtype dt; logits [T, N], topk_w, dgate [T, k]
 *   fp32; topk_idx, slot_row [T, k], counts [N] int32; dx_perm [max_rows, d]
 *   fp32; dhidden [T, d] fp32 out.  dx_shared [n_shared, T, d] fp32: the shared
 *   experts' input gradients (each one moe_expert_backward over all T rows of
 *   hidden with g_perm = dy and offsets {0, T}; P2 §3.3), or NULL with
 *   n_shared = 0.  Sums over tokens are taken in a fixed
 *   order (results do not depend on scheduling).
 *   ws  moe_workspace_size(MOE_OP_ROUTER_BACKWARD, T, d, N, k, f, dt) bytes.
 */
moe_status moe_router_backward(const void* hidden, const void* w_router, const float* logits,
                               const int32_t* topk_idx, const float* topk_w,
                               const int32_t* counts, const float* dgate, const float* dx_perm,
                               const int32_t* slot_row, const float* dx_shared, int n_shared,
                               float aux_coef, int T, int d, int N, int k, moe_dtype dt,
                               float* dhidden, float* dw_router, float* dbias, void* ws,
                               size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
