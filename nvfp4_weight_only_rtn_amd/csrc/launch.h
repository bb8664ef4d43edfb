// Host-side launchers implemented by the kernel translation units; called by attnq_api.hip
// after argument validation. Each returns the hipGetLastError() of its launches.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/attnq.h"

namespace attnq {

hipError_t launch_reconstruct(const attnq_theta& theta, uint16_t* W_eff, hipStream_t stream);
hipError_t launch_quantize(const attnq_theta& theta, uint8_t* codes, uint8_t* scales, float* tensor_scale,
                           hipStream_t stream);
// the same with W_eff rebuilt once into `workspace` (bf16 [N][K]) and quantized from there
hipError_t launch_quantize_staged(const attnq_theta& theta, uint8_t* codes, uint8_t* scales, float* tensor_scale,
                                  void* workspace, hipStream_t stream);
int64_t quantize_staged_workspace_bytes(int32_t N, int32_t K, int32_t r);
// the staged quantization of count (<= ATTNQ_MAX_BATCH) bundles, bundle i into codes[i], scales[i],
// tensor_scale[i] (its segment), W_eff at consecutive 256-byte-aligned places of `workspace`
hipError_t launch_quantize_staged_batch(const attnq_theta* theta, uint8_t* const* codes, uint8_t* const* scales,
                                        float* const* tensor_scale, int count, void* workspace, hipStream_t stream);
int64_t quantize_staged_batch_workspace_bytes(const attnq_theta* theta, int count);
hipError_t launch_gemv_nvfp4(const attnq_nvfp4& W, const uint16_t* x, float* y, hipStream_t stream);
// K split across workgroups for rows of 16384 elements or more (other shapes: launch_gemv_nvfp4);
// ws holds the tickets (zero on entry, zero again on exit) and the partial sums
hipError_t launch_gemv_nvfp4_splitk(const attnq_nvfp4& W, const uint16_t* x, float* y, void* ws, hipStream_t stream);
int64_t gemv_nvfp4_splitk_workspace_bytes(int N, int K);
// the same with the library's own per-device scratch (no allocation); the caller checks the size
hipError_t launch_gemv_nvfp4_splitk_noalloc(const attnq_nvfp4& W, const uint16_t* x, float* y, hipStream_t stream);
int64_t gemv_nvfp4_splitk_noalloc_max_bytes();
hipError_t launch_gemv_nvfp4_glu(const attnq_nvfp4& W, const uint16_t* x, int act, uint16_t* h, hipStream_t stream);
hipError_t launch_gemv_nvfp4_lowrank(const attnq_nvfp4& W, const uint16_t* s, const uint16_t* U, const uint16_t* V,
                                     int r, const uint16_t* x, float* ws, float* y, hipStream_t stream);
int64_t lowrank_workspace_floats(int K, int n_seg, int r);
hipError_t launch_gemv_nvfp4_lowrank_splitk(const attnq_nvfp4& W, const uint16_t* s, const uint16_t* U,
                                            const uint16_t* V, int r, const uint16_t* x, float* ws, void* split_ws,
                                            float* y, hipStream_t stream);
// streaming read of two byte ranges (multiples of 16 bytes), nothing written: the read ceiling
hipError_t launch_read_ceiling(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes, uint32_t* sink,
                               hipStream_t stream);
hipError_t launch_gemv_bf16(const uint16_t* W, int N, int K, const uint16_t* x, float* y, hipStream_t stream);
hipError_t launch_gemm_nvfp4_small_m(const attnq_nvfp4& W, const uint16_t* X, int M, int ldx, float* Y, int ldy,
                                     hipStream_t stream);
// the same with K cut into one-shot slices on separate workgroups (workspace: fixed ticket area, then
// the slices' partial sums); shapes without slices run launch_gemm_nvfp4_small_m
hipError_t launch_gemm_nvfp4_small_m_splitk(const attnq_nvfp4& W, const uint16_t* X, int M, int ldx, float* Y, int ldy,
                                            void* ws, hipStream_t stream);
int64_t gemm_small_m_splitk_workspace_bytes(int N, int K, int M);
// M = 1 .. 4 on the batch-1 walk for rows of at most 192 chunks; false (nothing launched) otherwise
bool launch_gemm_nvfp4_tokens(const attnq_nvfp4& W, const uint16_t* X, int M, int ldx, float* Y, int ldy,
                              hipStream_t stream);

}  // namespace attnq
