// C ABI of libmoe_mi355x.so: argument validation on the host (before any HIP
// call), then the launchers of each step.  Declarations and the contract of
// every entry point are in include/moe.h.
#include "moe.h"

#include <cmath>
#include <cstdint>
#include <initializer_list>

#include "internal.hpp"

namespace {

constexpr int kMaxExperts = 256;

inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }
inline bool dtype_ok(moe_dtype dt) { return dt == MOE_F32 || dt == MOE_BF16; }
inline int elem_bytes(moe_dtype dt) { return dt == MOE_BF16 ? 2 : 4; }
inline moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Every device buffer must be 16-byte aligned: the kernels read and write them
// with 16-byte vector and buffer accesses (hipMalloc and torch allocations are
// 256-byte aligned).  Null pointers pass here; the null checks are separate.
inline bool aligned16(std::initializer_list<const void*> ps) {
  for (const void* q : ps)
    if (reinterpret_cast<uintptr_t>(q) & 15) return false;
  return true;
}

// Shared shape checks.  Order: invalid (nonsense) arguments first, then
// unsupported-but-meaningful ones.
moe_status check_tnk(int T, int N, int k) {
  if (T < 1 || N < 1 || k < 1 || k > N) return MOE_ERR_INVALID_ARG;
  if (N > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(T) * k >= (int64_t{1} << 31)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status check_d(int d) {
  if (d < 1) return MOE_ERR_INVALID_ARG;
  if (d % 64 != 0) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status check_expert_shape(int N, int d, int f, int max_rows, moe_dtype dt) {
  if (N < 1 || d < 1 || f < 1 || max_rows < 1) return MOE_ERR_INVALID_ARG;
  if (!dtype_ok(dt)) return MOE_ERR_UNSUPPORTED;
  if (N > kMaxExperts || d % 64 != 0 || f % 64 != 0) return MOE_ERR_UNSUPPORTED;
  if (dt == MOE_BF16 && (d % 256 != 0 || f % 128 != 0)) return MOE_ERR_UNSUPPORTED;
  // the down projection stores a 256-row fp32 tile of y_perm through a buffer
  // resource with 32-bit offsets
  if (dt == MOE_BF16 && d >= (1 << 21)) return MOE_ERR_UNSUPPORTED;
  // one expert matrix is addressed through a buffer resource with a 31-bit byte range
  if (static_cast<int64_t>(d) * f * elem_bytes(dt) >= (int64_t{1} << 31)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Capacity C = floor((T*k)/N * CF) in double, CF <= 0 meaning "no limit".  CF
// arrives as a double: narrowed to float, a factor such as 1.05 rounds below
// its decimal value and C can come out one short wherever (T*k)/N * CF is a
// whole number.
int capacity_of(int T, int k, int N, double cf) {
  if (!(cf > 0.0)) return T;
  const double c = std::floor((static_cast<double>(T) * k) / N * cf);
  if (c >= static_cast<double>(T)) return T;
  return static_cast<int>(c);
}

// Activations held in the moe_expert_ffn workspace, padded to 256 bytes.
size_t act_bytes(int rows, int f, moe_dtype dt) {
  const size_t b = static_cast<size_t>(rows) * static_cast<size_t>(f) * elem_bytes(dt);
  return (b + 255) & ~static_cast<size_t>(255);
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: shape or dtype outside the supported limits";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: HIP launch error";
  }
  return "unknown moe_status";
}

int moe_capacity(int T, int k, int N, double capacity_factor) {
  if (T < 1 || N < 1 || k < 1 || k > N || std::isnan(capacity_factor)) return -1;
  return capacity_of(T, k, N, capacity_factor);
}

size_t moe_workspace_size(moe_op op, int T, int d, int N, int k, int f, moe_dtype dt) {
  if (T < 1 || N < 1 || k < 1) return 0;
  switch (op) {
    case MOE_OP_ROUTE:
      if (d < 1 || !dtype_ok(dt)) return 0;
      return dt == MOE_BF16 ? moe::route_ws_bytes(T, d, N) : 0;
    case MOE_OP_PERMUTE: return moe::permute_ws_bytes(T, N);
    case MOE_OP_PERMUTE_REROUTE:
      if (N > kMaxExperts || static_cast<int64_t>(T) * k >= (int64_t{1} << 31)) return 0;
      return moe::permute_reroute_ws_bytes(T, N, k);
    case MOE_OP_EXPERT_FFN:
      if (d < 1 || f < 1 || !dtype_ok(dt)) return 0;
      return act_bytes(T * k, f, dt) +
             moe::expert_down_ws_bytes(N, d, f, T * k, dt == MOE_BF16);
    case MOE_OP_EXPERT_DOWN:
      if (d < 1 || f < 1 || !dtype_ok(dt)) return 0;
      return moe::expert_down_ws_bytes(N, d, f, T * k, dt == MOE_BF16);
    case MOE_OP_AUX_LOSS: return moe::aux_ws_bytes(T, N);
    case MOE_OP_EXPERT_BACKWARD:
      if (d < 1 || f < 1 || !dtype_ok(dt)) return 0;
      return moe::expert_backward_ws_bytes(d, f, T * k, dt == MOE_BF16);
    case MOE_OP_EXPERT_BACKWARD_SAVED:
      if (d < 1 || f < 1 || !dtype_ok(dt)) return 0;
      return moe::expert_backward_saved_ws_bytes(d, f, T * k, dt == MOE_BF16);
    case MOE_OP_ROUTER_BACKWARD:
      if (d < 1 || N > kMaxExperts) return 0;
      return moe::router_backward_ws_bytes(T, d, N);
    default: return 0;
  }
}

moe_status moe_route(const void* hidden, const void* w_router, const float* bias, int T, int d,
                     int N, int k, moe_dtype dt, float* logits, int32_t* topk_idx, float* topk_w,
                     int32_t* counts, void* ws, size_t ws_bytes, void* stream) {
  if (!aligned16({hidden, w_router, bias, logits, topk_idx, topk_w, counts, ws})) return MOE_ERR_INVALID_ARG;
  if (!hidden || !w_router || !logits || !topk_idx || !topk_w || !counts) return MOE_ERR_INVALID_ARG;
  moe_status s = check_tnk(T, N, k);
  if (s != MOE_OK) return s;
  if ((s = check_d(d)) != MOE_OK) return s;
  if (!dtype_ok(dt)) return MOE_ERR_UNSUPPORTED;
  const size_t need = dt == MOE_BF16 ? moe::route_ws_bytes(T, d, N) : 0;
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  if (need > 0 && !ws) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_route(hidden, w_router, bias, T, d, N, k, dt == MOE_BF16, logits,
                                      topk_idx, topk_w, counts, ws, as_stream(stream)));
}

moe_status moe_permute(const void* hidden, const int32_t* topk_idx, int T, int d, int N, int k,
                       double capacity_factor, moe_dtype dt, void* x_perm, int32_t* perm_src,
                       int32_t* slot_row, int32_t* kept, int32_t* offsets, void* ws,
                       size_t ws_bytes, void* stream) {
  if (!aligned16({hidden, topk_idx, x_perm, perm_src, slot_row, kept, offsets, ws})) return MOE_ERR_INVALID_ARG;
  if (!hidden || !topk_idx || !x_perm || !perm_src || !slot_row || !kept || !offsets)
    return MOE_ERR_INVALID_ARG;
  if (std::isnan(capacity_factor)) return MOE_ERR_INVALID_ARG;
  moe_status s = check_tnk(T, N, k);
  if (s != MOE_OK) return s;
  if ((s = check_d(d)) != MOE_OK) return s;
  if (!dtype_ok(dt)) return MOE_ERR_UNSUPPORTED;
  const size_t need = moe::permute_ws_bytes(T, N);
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  if (!ws) return MOE_ERR_INVALID_ARG;
  const int C = capacity_of(T, k, N, capacity_factor);
  return hip_status(moe::launch_permute(hidden, topk_idx, T, d, N, k, C, elem_bytes(dt), x_perm,
                                        perm_src, slot_row, kept, offsets, ws, as_stream(stream)));
}

moe_status moe_permute_noalloc(const void* hidden, const int32_t* topk_idx, int T, int d, int N,
                               int k, double capacity_factor, moe_dtype dt, void* x_perm,
                               int32_t* perm_src, int32_t* slot_row, int32_t* kept,
                               int32_t* offsets, void* stream) {
  if (!aligned16({hidden, topk_idx, x_perm, perm_src, slot_row, kept, offsets})) return MOE_ERR_INVALID_ARG;
  if (!hidden || !topk_idx || !x_perm || !perm_src || !slot_row || !kept || !offsets)
    return MOE_ERR_INVALID_ARG;
  if (std::isnan(capacity_factor)) return MOE_ERR_INVALID_ARG;
  moe_status s = check_tnk(T, N, k);
  if (s != MOE_OK) return s;
  if ((s = check_d(d)) != MOE_OK) return s;
  if (!dtype_ok(dt)) return MOE_ERR_UNSUPPORTED;
  static_assert(MOE_PERMUTE_NOALLOC_SCRATCH_BYTES == moe::kPermuteNoAllocScratchBytes,
                "header and library disagree on the static scratch size");
  if (moe::permute_ws_bytes(T, N) > moe::kPermuteNoAllocScratchBytes) return MOE_ERR_WORKSPACE;
  const int C = capacity_of(T, k, N, capacity_factor);
  return hip_status(moe::launch_permute_noalloc(hidden, topk_idx, T, d, N, k, C, elem_bytes(dt),
                                                x_perm, perm_src, slot_row, kept, offsets,
                                                as_stream(stream)));
}

moe_status moe_permute_reroute(const void* hidden, const int32_t* topk_idx, const float* logits,
                               int T, int d, int N, int k, double capacity_factor, moe_dtype dt,
                               void* x_perm, int32_t* perm_src, int32_t* slot_row, int32_t* kept,
                               int32_t* offsets, void* ws, size_t ws_bytes, void* stream) {
  if (!aligned16({hidden, topk_idx, logits, x_perm, perm_src, slot_row, kept, offsets, ws})) return MOE_ERR_INVALID_ARG;
  if (!hidden || !topk_idx || !logits || !x_perm || !perm_src || !slot_row || !kept || !offsets)
    return MOE_ERR_INVALID_ARG;
  if (std::isnan(capacity_factor)) return MOE_ERR_INVALID_ARG;
  moe_status s = check_tnk(T, N, k);
  if (s != MOE_OK) return s;
  if ((s = check_d(d)) != MOE_OK) return s;
  if (!dtype_ok(dt)) return MOE_ERR_UNSUPPORTED;
  const size_t need = moe::permute_reroute_ws_bytes(T, N, k);
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  if (!ws) return MOE_ERR_INVALID_ARG;
  const int C = capacity_of(T, k, N, capacity_factor);
  return hip_status(moe::launch_permute_reroute(hidden, topk_idx, logits, T, d, N, k, C,
                                                elem_bytes(dt), x_perm, perm_src, slot_row, kept,
                                                offsets, ws, as_stream(stream)));
}

moe_status moe_expert_up(const void* x_perm, const int32_t* offsets, const void* w1,
                         const void* w3, int N, int d, int f, int max_rows, moe_dtype dt,
                         void* act, void* stream) {
  if (!aligned16({x_perm, offsets, w1, w3, act})) return MOE_ERR_INVALID_ARG;
  if (!x_perm || !offsets || !w1 || !w3 || !act) return MOE_ERR_INVALID_ARG;
  moe_status s = check_expert_shape(N, d, f, max_rows, dt);
  if (s != MOE_OK) return s;
  return hip_status(moe::launch_expert_up(x_perm, offsets, w1, w3, N, d, f, max_rows,
                                          dt == MOE_BF16, act, nullptr, as_stream(stream)));
}

moe_status moe_expert_up_save(const void* x_perm, const int32_t* offsets, const void* w1,
                              const void* w3, int N, int d, int f, int max_rows, moe_dtype dt,
                              void* act, void* h13, void* stream) {
  if (!aligned16({x_perm, offsets, w1, w3, act, h13})) return MOE_ERR_INVALID_ARG;
  if (!x_perm || !offsets || !w1 || !w3 || !act || !h13) return MOE_ERR_INVALID_ARG;
  moe_status s = check_expert_shape(N, d, f, max_rows, dt);
  if (s != MOE_OK) return s;
  return hip_status(moe::launch_expert_up(x_perm, offsets, w1, w3, N, d, f, max_rows,
                                          dt == MOE_BF16, act, h13, as_stream(stream)));
}

moe_status moe_expert_down(const void* act, const int32_t* offsets, const void* w2, int N, int d,
                           int f, int max_rows, moe_dtype dt, float* y_perm, void* ws,
                           size_t ws_bytes, void* stream) {
  if (!aligned16({act, offsets, w2, y_perm, ws})) return MOE_ERR_INVALID_ARG;
  if (!act || !offsets || !w2 || !y_perm) return MOE_ERR_INVALID_ARG;
  moe_status s = check_expert_shape(N, d, f, max_rows, dt);
  if (s != MOE_OK) return s;
  const size_t need = moe::expert_down_ws_bytes(N, d, f, max_rows, dt == MOE_BF16);
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  if (need > 0 && !ws) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_expert_down(act, offsets, w2, N, d, f, max_rows, dt == MOE_BF16,
                                            y_perm, need > 0 ? ws : nullptr, as_stream(stream)));
}

moe_status moe_expert_ffn(const void* x_perm, const int32_t* offsets, const void* w1,
                          const void* w3, const void* w2, int N, int d, int f, int max_rows,
                          moe_dtype dt, float* y_perm, void* ws, size_t ws_bytes, void* stream) {
  if (!aligned16({x_perm, offsets, w1, w3, w2, y_perm, ws})) return MOE_ERR_INVALID_ARG;
  if (!x_perm || !offsets || !w1 || !w3 || !w2 || !y_perm) return MOE_ERR_INVALID_ARG;
  moe_status s = check_expert_shape(N, d, f, max_rows, dt);
  if (s != MOE_OK) return s;
  const size_t need_act = act_bytes(max_rows, f, dt);
  const size_t need_down = moe::expert_down_ws_bytes(N, d, f, max_rows, dt == MOE_BF16);
  if (ws_bytes < need_act + need_down) return MOE_ERR_WORKSPACE;
  if (!ws) return MOE_ERR_INVALID_ARG;
  hipError_t e = moe::launch_expert_up(x_perm, offsets, w1, w3, N, d, f, max_rows, dt == MOE_BF16,
                                       ws, nullptr, as_stream(stream));
  if (e != hipSuccess) return MOE_ERR_HIP;
  void* down_ws = need_down > 0 ? static_cast<char*>(ws) + need_act : nullptr;
  return hip_status(moe::launch_expert_down(ws, offsets, w2, N, d, f, max_rows, dt == MOE_BF16,
                                            y_perm, down_ws, as_stream(stream)));
}

moe_status moe_quantize_fp8(const void* w, moe_dtype dt, int N, int K, int M, uint8_t* q,
                            float* scale, void* stream) {
  if (!aligned16({w, q, scale})) return MOE_ERR_INVALID_ARG;
  if (!w || !q || !scale) return MOE_ERR_INVALID_ARG;
  if (N < 1 || K < 1 || M < 1) return MOE_ERR_INVALID_ARG;
  if (!dtype_ok(dt)) return MOE_ERR_UNSUPPORTED;
  if (N > 65535) return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_quantize_fp8(w, dt == MOE_BF16, N, K, M, q, scale,
                                             as_stream(stream)));
}

// FP8 weights run on the weight-streaming kernels only: bf16 activations,
// the bf16 shape limits, and at most 32 rows per expert on average.
static moe_status check_fp8_shape(int N, int d, int f, int max_rows) {
  moe_status s = check_expert_shape(N, d, f, max_rows, MOE_BF16);
  if (s != MOE_OK) return s;
  if (!moe::fp8_rows_supported(max_rows, N)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status moe_expert_up_fp8(const void* x_perm, const int32_t* offsets, const uint8_t* w1q,
                             const uint8_t* w3q, const float* s1, const float* s3, int N, int d,
                             int f, int max_rows, void* act, void* stream) {
  if (!aligned16({x_perm, offsets, w1q, w3q, s1, s3, act})) return MOE_ERR_INVALID_ARG;
  if (!x_perm || !offsets || !w1q || !w3q || !s1 || !s3 || !act) return MOE_ERR_INVALID_ARG;
  moe_status s = check_fp8_shape(N, d, f, max_rows);
  if (s != MOE_OK) return s;
  return hip_status(moe::launch_expert_up_fp8(x_perm, offsets, w1q, w3q, s1, s3, N, d, f,
                                              max_rows, act, as_stream(stream)));
}

moe_status moe_expert_down_fp8(const void* act, const int32_t* offsets, const uint8_t* w2q,
                               const float* s2, int N, int d, int f, int max_rows, float* y_perm,
                               void* stream) {
  if (!aligned16({act, offsets, w2q, s2, y_perm})) return MOE_ERR_INVALID_ARG;
  if (!act || !offsets || !w2q || !s2 || !y_perm) return MOE_ERR_INVALID_ARG;
  moe_status s = check_fp8_shape(N, d, f, max_rows);
  if (s != MOE_OK) return s;
  return hip_status(moe::launch_expert_down_fp8(act, offsets, w2q, s2, N, d, f, max_rows, y_perm,
                                                as_stream(stream)));
}

moe_status moe_combine(const float* y_perm, const int32_t* slot_row, const float* topk_w,
                       const float* y_shared, int n_shared, int T, int d, int k, moe_dtype dt,
                       void* y, void* stream) {
  if (!aligned16({y_perm, slot_row, topk_w, y_shared, y})) return MOE_ERR_INVALID_ARG;
  if (!y_perm || !slot_row || !topk_w || !y) return MOE_ERR_INVALID_ARG;
  if (T < 1 || k < 1 || n_shared < 0 || (n_shared > 0 && !y_shared)) return MOE_ERR_INVALID_ARG;
  if (k > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  moe_status s = check_d(d);
  if (s != MOE_OK) return s;
  if (!dtype_ok(dt)) return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_combine(y_perm, slot_row, topk_w, n_shared > 0 ? y_shared : nullptr,
                                        n_shared, T, d, k, dt == MOE_BF16, y, as_stream(stream)));
}

moe_status moe_aux_loss(const float* logits, const int32_t* counts, int T, int N, int k,
                        float* aux, void* ws, size_t ws_bytes, void* stream) {
  if (!aligned16({logits, counts, aux, ws})) return MOE_ERR_INVALID_ARG;
  if (!logits || !counts || !aux) return MOE_ERR_INVALID_ARG;
  moe_status s = check_tnk(T, N, k);
  if (s != MOE_OK) return s;
  if (ws_bytes < moe::aux_ws_bytes(T, N)) return MOE_ERR_WORKSPACE;
  if (!ws) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_aux(logits, counts, T, N, k, aux, ws, as_stream(stream)));
}

moe_status moe_combine_backward(const void* dy, const float* y_perm, const int32_t* slot_row,
                                const float* topk_w, int T, int d, int k, moe_dtype dt,
                                void* g_perm, float* dgate, void* stream) {
  if (!aligned16({dy, y_perm, slot_row, topk_w, g_perm, dgate})) return MOE_ERR_INVALID_ARG;
  if (!dy || !y_perm || !slot_row || !topk_w || !g_perm || !dgate) return MOE_ERR_INVALID_ARG;
  if (T < 1 || k < 1) return MOE_ERR_INVALID_ARG;
  if (k > kMaxExperts || static_cast<int64_t>(T) * k >= (int64_t{1} << 31)) return MOE_ERR_UNSUPPORTED;
  moe_status s = check_d(d);
  if (s != MOE_OK) return s;
  if (!dtype_ok(dt)) return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_combine_backward(dy, y_perm, slot_row, topk_w, T, d, k,
                                                 dt == MOE_BF16, g_perm, dgate, as_stream(stream)));
}

moe_status moe_expert_backward(const void* x_perm, const void* g_perm, const int32_t* offsets,
                               const void* w1, const void* w3, const void* w2, int N, int d,
                               int f, int max_rows, moe_dtype dt, float* dx_perm, float* dw1,
                               float* dw3, float* dw2, void* ws, size_t ws_bytes, void* stream) {
  if (!aligned16({x_perm, g_perm, offsets, w1, w3, w2, dx_perm, dw1, dw3, dw2, ws})) return MOE_ERR_INVALID_ARG;
  if (!x_perm || !g_perm || !offsets || !w1 || !w3 || !w2 || !dx_perm || !dw1 || !dw3 || !dw2)
    return MOE_ERR_INVALID_ARG;
  moe_status s = check_expert_shape(N, d, f, max_rows, dt);
  if (s != MOE_OK) return s;
  // bf16: 256-column tiles over f, and 31-bit buffer ranges over an expert's rows of
  // [dh1 | dh3] ([rows, 2f]) and of x_perm / g_perm ([rows, d])
  if (dt == MOE_BF16 && (f % 256 != 0 ||
                         static_cast<int64_t>(max_rows) * f >= (int64_t{1} << 29) ||
                         static_cast<int64_t>(max_rows) * d >= (int64_t{1} << 30)))
    return MOE_ERR_UNSUPPORTED;
  const size_t need = moe::expert_backward_ws_bytes(d, f, max_rows, dt == MOE_BF16);
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  if (!ws) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_expert_backward(x_perm, g_perm, offsets, w1, w3, w2, N, d, f,
                                                max_rows, dt == MOE_BF16, dx_perm, dw1, dw3, dw2,
                                                ws, as_stream(stream)));
}

moe_status moe_expert_backward_saved(const void* x_perm, const void* g_perm, const void* h13,
                                     const void* act, const int32_t* offsets, const void* w1,
                                     const void* w3, const void* w2, int N, int d, int f,
                                     int max_rows, moe_dtype dt, float* dx_perm, float* dw1,
                                     float* dw3, float* dw2, void* ws, size_t ws_bytes,
                                     void* stream) {
  if (!aligned16({x_perm, g_perm, h13, act, offsets, w1, w3, w2, dx_perm, dw1, dw3, dw2, ws})) return MOE_ERR_INVALID_ARG;
  if (!x_perm || !g_perm || !h13 || !offsets || !w1 || !w3 || !w2 || !dx_perm || !dw1 || !dw3 ||
      !dw2)
    return MOE_ERR_INVALID_ARG;
  moe_status s = check_expert_shape(N, d, f, max_rows, dt);
  if (s != MOE_OK) return s;
  if (dt == MOE_BF16 && (f % 256 != 0 ||
                         static_cast<int64_t>(max_rows) * f >= (int64_t{1} << 29) ||
                         static_cast<int64_t>(max_rows) * d >= (int64_t{1} << 30)))
    return MOE_ERR_UNSUPPORTED;
  const size_t need = moe::expert_backward_saved_ws_bytes(d, f, max_rows, dt == MOE_BF16);
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  if (!ws) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_expert_backward_saved(x_perm, g_perm, h13, act, offsets, w1, w3,
                                                      w2, N, d, f, max_rows, dt == MOE_BF16,
                                                      dx_perm, dw1, dw3, dw2, ws,
                                                      as_stream(stream)));
}

moe_status moe_router_backward(const void* hidden, const void* w_router, const float* logits,
                               const int32_t* topk_idx, const float* topk_w,
                               const int32_t* counts, const float* dgate, const float* dx_perm,
                               const int32_t* slot_row, const float* dx_shared, int n_shared,
                               float aux_coef, int T, int d, int N, int k, moe_dtype dt,
                               float* dhidden, float* dw_router, float* dbias, void* ws,
                               size_t ws_bytes, void* stream) {
  if (!aligned16({hidden, w_router, logits, topk_idx, topk_w, counts, dgate, dx_perm, slot_row, dx_shared, dhidden, dw_router, dbias, ws})) return MOE_ERR_INVALID_ARG;
  if (!hidden || !w_router || !logits || !topk_idx || !topk_w || !counts || !dgate || !dx_perm ||
      !slot_row || !dhidden || !dw_router)
    return MOE_ERR_INVALID_ARG;
  if (n_shared < 0 || (n_shared > 0 && !dx_shared)) return MOE_ERR_INVALID_ARG;
  if (std::isnan(aux_coef)) return MOE_ERR_INVALID_ARG;
  moe_status s = check_tnk(T, N, k);
  if (s != MOE_OK) return s;
  if ((s = check_d(d)) != MOE_OK) return s;
  if (!dtype_ok(dt)) return MOE_ERR_UNSUPPORTED;
  const size_t need = moe::router_backward_ws_bytes(T, d, N);
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  if (!ws) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_router_backward(hidden, w_router, logits, topk_idx, topk_w,
                                                counts, dgate, dx_perm, slot_row,
                                                n_shared > 0 ? dx_shared : nullptr, n_shared,
                                                aux_coef, T, d, N, k, dt == MOE_BF16, dhidden,
                                                dw_router, dbias, ws, as_stream(stream)));
}

}  // extern "C"
