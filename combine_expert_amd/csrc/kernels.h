// kernels.h -- launchers shared between the C ABI (api.hip) and the kernel
// translation units.  Arguments are already validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

hipError_t launch_update_expert(const int32_t *ids, const float *scores, const int32_t *table,
                                const float *thr, const uint8_t *token_mask, int Bs, int K,
                                int n_logical, int F, int n_instances, int32_t *out_ids,
                                uint8_t *out_mask, int32_t *dev_err, hipStream_t stream);

hipError_t launch_dispatch(const uint16_t *x, const int32_t *ids, const uint8_t *mask,
                           const uint8_t *token_mask, int Bs, int H, int K, int E,
                           int quant_mode, int tile, const float *qs,
                           int qs_kind, void *expand_x, void *expand_scales, int32_t *counts,
                           int32_t *offsets, int32_t *expand_src, int32_t *assist_dst,
                           int32_t *dev_err, hipStream_t stream);

hipError_t launch_update_dispatch(const uint16_t *x, const int32_t *ids, const float *scores,
                                  const int32_t *table, const float *thr,
                                  const uint8_t *token_mask, int n_logical, int F, int Bs, int H,
                                  int K, int E, int quant_mode, int tile, const float *qs,
                                  int qs_kind, int32_t *balanced_ids, uint8_t *balanced_mask,
                                  void *expand_x, void *expand_scales, int32_t *counts,
                                  int32_t *offsets, int32_t *expand_src, int32_t *assist_dst,
                                  int32_t *dev_err, hipStream_t stream);

hipError_t launch_combine(const uint16_t *expert_out, const int32_t *assist,
                          const float *scales, const uint16_t *shared,
                          const uint16_t *residual, const uint16_t *gamma, float eps, int Bs,
                          int H, int K, int shared_mode, uint16_t *y, uint16_t *x_out,
                          float *rstd, int32_t *dev_err, hipStream_t stream);

hipError_t launch_expert_gemm(int quant_mode, const void *a, const void *a_sc,
                              const int32_t *offsets, int E, int rows, const void *w,
                              const void *w_sc, int N, int K, uint16_t *y, int32_t *dev_err,
                              hipStream_t stream);

hipError_t launch_expert_swiglu(const uint16_t *y1, const int32_t *offsets, int E, int rows,
                                int I, bool group_major, uint8_t *codes, uint8_t *sc,
                                uint16_t *act, int32_t *dev_err, hipStream_t stream);

// Threads per row block: one thread per 16 row elements, rounded up to
// whole waves (64 .. 512 threads for H in [1024, 8192]).  Kernels derive
// their block size from H with these functions instead of reading blockDim,
// whose value is fetched through a chain of dependent loads.
__host__ __device__ inline int row_threads(int H) { return ((H / 16 + 63) / 64) * 64; }

// Threads per dispatch block: the row's threads and one more wave.
__host__ __device__ inline int dispatch_threads(int H) { return row_threads(H) + 64; }

}  // namespace moe
