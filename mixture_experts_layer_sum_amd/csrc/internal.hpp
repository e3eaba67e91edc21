// Launchers behind the C ABI (one per step of the layer).  Each enqueues its
// kernels on `stream` and returns hipGetLastError(); the API layer has
// already validated every argument.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

size_t route_ws_bytes(int T, int d, int N);   // bf16 router k-split partials (0 if none)
hipError_t launch_route(const void* hidden, const void* w_router, const float* bias, int T, int d,
                        int N, int k, bool bf16, float* logits, int32_t* topk_idx, float* topk_w,
                        int32_t* counts, void* ws, hipStream_t stream);

size_t permute_ws_bytes(int T, int N);
hipError_t launch_permute(const void* hidden, const int32_t* topk_idx, int T, int d, int N, int k,
                          int C, int elem_bytes, void* x_perm, int32_t* perm_src,
                          int32_t* slot_row, int32_t* kept, int32_t* offsets, void* ws,
                          hipStream_t stream);

// moe_permute_noalloc: the chunk tables live in a static device array of this size
constexpr size_t kPermuteNoAllocScratchBytes = size_t{4} << 20;
hipError_t launch_permute_noalloc(const void* hidden, const int32_t* topk_idx, int T, int d, int N,
                                  int k, int C, int elem_bytes, void* x_perm, int32_t* perm_src,
                                  int32_t* slot_row, int32_t* kept, int32_t* offsets,
                                  hipStream_t stream);

size_t permute_reroute_ws_bytes(int T, int N, int k);
hipError_t launch_permute_reroute(const void* hidden, const int32_t* topk_idx,
                                  const float* logits, int T, int d, int N, int k, int C,
                                  int elem_bytes, void* x_perm, int32_t* perm_src,
                                  int32_t* slot_row, int32_t* kept, int32_t* offsets, void* ws,
                                  hipStream_t stream);

// h13: NULL, or [max_rows, 2f] in the layer dtype: h1 = x W1 then h3 = x W3 per row
hipError_t launch_expert_up(const void* x_perm, const int32_t* offsets, const void* w1,
                            const void* w3, int N, int d, int f, int max_rows, bool bf16,
                            void* act, void* h13, hipStream_t stream);
size_t expert_down_ws_bytes(int N, int d, int f, int max_rows, bool bf16);   // current device
hipError_t launch_expert_down(const void* act, const int32_t* offsets, const void* w2, int N,
                              int d, int f, int max_rows, bool bf16, float* y_perm, void* ws,
                              hipStream_t stream);

hipError_t launch_quantize_fp8(const void* w, bool bf16, int N, int K, int M, uint8_t* q,
                               float* scale, hipStream_t stream);
bool fp8_rows_supported(int max_rows, int N);
hipError_t launch_expert_up_fp8(const void* x_perm, const int32_t* offsets, const uint8_t* w1q,
                                const uint8_t* w3q, const float* s1, const float* s3, int N,
                                int d, int f, int max_rows, void* act, hipStream_t stream);
hipError_t launch_expert_down_fp8(const void* act, const int32_t* offsets, const uint8_t* w2q,
                                  const float* s2, int N, int d, int f, int max_rows,
                                  float* y_perm, hipStream_t stream);

hipError_t launch_combine(const float* y_perm, const int32_t* slot_row, const float* topk_w,
                          const float* y_shared, int n_shared, int T, int d, int k, bool bf16,
                          void* y, hipStream_t stream);

size_t aux_ws_bytes(int T, int N);
hipError_t launch_aux(const float* logits, const int32_t* counts, int T, int N, int k, float* aux,
                      void* ws, hipStream_t stream);

hipError_t launch_combine_backward(const void* dy, const float* y_perm, const int32_t* slot_row,
                                   const float* topk_w, int T, int d, int k, bool bf16,
                                   void* g_perm, float* dgate, hipStream_t stream);
size_t expert_backward_ws_bytes(int d, int f, int max_rows, bool bf16);
size_t expert_backward_saved_ws_bytes(int d, int f, int max_rows, bool bf16);
// Compute units of the current device (0 if there is none).
int device_cus();

hipError_t launch_expert_backward_saved(const void* x_perm, const void* g_perm, const void* h13,
                                        const void* act_in, const int32_t* offsets,
                                        const void* w1, const void* w3,
                                        const void* w2, int N, int d, int f, int max_rows,
                                        bool bf16, float* dx_perm, float* dw1, float* dw3,
                                        float* dw2, void* ws, hipStream_t stream);
hipError_t launch_expert_backward(const void* x_perm, const void* g_perm, const int32_t* offsets,
                                  const void* w1, const void* w3, const void* w2, int N, int d,
                                  int f, int max_rows, bool bf16, float* dx_perm, float* dw1,
                                  float* dw3, float* dw2, void* ws, hipStream_t stream);
size_t router_backward_ws_bytes(int T, int d, int N);
hipError_t launch_router_backward(const void* hidden, const void* w_router, const float* logits,
                                  const int32_t* topk_idx, const float* topk_w,
                                  const int32_t* counts, const float* dgate, const float* dx_perm,
                                  const int32_t* slot_row, const float* dx_shared, int n_shared,
                                  float aux_coef, int T, int d, int N, int k, bool bf16,
                                  float* dhidden, float* dw_router, float* dbias, void* ws,
                                  hipStream_t stream);

}  // namespace moe
