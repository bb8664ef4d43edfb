// C ABI of libattnq.so: host-side argument validation, then the kernel launchers.
// Validation touches no device memory and makes no HIP call, so every error path below can
// be exercised on a machine without a GPU.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/attnq.h"
#include "launch.h"

namespace {

constexpr int32_t kMaxRank = 64;
constexpr int32_t kMaxM = 16;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// A pointer to an empty array (N == 0) may be NULL; everything else must be non-NULL.
attnq_status check_theta(const attnq_theta* t) {
  if (t == nullptr) return ATTNQ_ERR_NULL;
  if (t->W0 == nullptr && t->N != 0) return ATTNQ_ERR_NULL;
  if (t->N < 0 || t->K <= 0 || t->K % 32 != 0 || t->r < 0 || t->r > kMaxRank) return ATTNQ_ERR_SHAPE;
  if (t->r > 0 && (t->U == nullptr || t->V == nullptr)) return ATTNQ_ERR_NULL;
  if (!aligned(t->W0, 16)) return ATTNQ_ERR_ALIGN;
  if (t->s && !aligned(t->s, 2)) return ATTNQ_ERR_ALIGN;
  if (t->r > 0 && (!aligned(t->U, 2) || !aligned(t->V, 2))) return ATTNQ_ERR_ALIGN;
  return ATTNQ_OK;
}

attnq_status check_nvfp4(const attnq_nvfp4* w) {
  if (w == nullptr || w->tensor_scale == nullptr) return ATTNQ_ERR_NULL;
  if ((w->codes == nullptr || w->scales == nullptr) && w->N != 0) return ATTNQ_ERR_NULL;
  if (w->layout != ATTNQ_LAYOUT_ROW_MAJOR) return ATTNQ_ERR_LAYOUT;
  if (w->N < 0 || w->K <= 0 || w->K % 32 != 0) return ATTNQ_ERR_SHAPE;
  // codes and scales are addressed with 32-bit byte offsets inside the kernels
  if ((int64_t)w->N * (w->K / 2) > (int64_t{1} << 32)) return ATTNQ_ERR_SHAPE;
  if (w->n_seg < 1 || w->n_seg > ATTNQ_MAX_SEGMENTS) return ATTNQ_ERR_SEGMENT;
  int32_t prev = 0;
  for (int i = 0; i < w->n_seg; ++i) {
    if (w->seg_end[i] <= prev && !(w->N == 0 && w->n_seg == 1)) return ATTNQ_ERR_SEGMENT;
    prev = w->seg_end[i];
  }
  if (w->seg_end[w->n_seg - 1] != w->N) return ATTNQ_ERR_SEGMENT;
  if (!aligned(w->codes, 16) || !aligned(w->scales, 4) || !aligned(w->tensor_scale, 4)) return ATTNQ_ERR_ALIGN;
  return ATTNQ_OK;
}

attnq_status from_hip(hipError_t e) { return e == hipSuccess ? ATTNQ_OK : ATTNQ_ERR_HIP; }

}  // namespace

extern "C" {

attnq_status attnq_reconstruct(const attnq_theta* theta, uint16_t* W_eff, attnq_stream stream) {
  attnq_status st = check_theta(theta);
  if (st != ATTNQ_OK) return st;
  if (W_eff == nullptr && theta->N != 0) return ATTNQ_ERR_NULL;
  if (!aligned(W_eff, 16)) return ATTNQ_ERR_ALIGN;
  return from_hip(attnq::launch_reconstruct(*theta, W_eff, static_cast<hipStream_t>(stream)));
}

attnq_status attnq_quantize_nvfp4(const attnq_theta* theta, const attnq_nvfp4* dst, int32_t seg, attnq_stream stream) {
  attnq_status st = check_theta(theta);
  if (st != ATTNQ_OK) return st;
  st = check_nvfp4(dst);
  if (st != ATTNQ_OK) return st;
  if (theta->K != dst->K) return ATTNQ_ERR_SHAPE;
  if (seg < 0 || seg >= dst->n_seg) return ATTNQ_ERR_SEGMENT;
  const int32_t start = seg == 0 ? 0 : dst->seg_end[seg - 1];
  if (dst->seg_end[seg] - start != theta->N) return ATTNQ_ERR_SEGMENT;
  uint8_t* codes = dst->codes + (size_t)start * (dst->K / 2);
  uint8_t* scales = dst->scales + (size_t)start * (dst->K / 16);
  return from_hip(attnq::launch_quantize(*theta, codes, scales, dst->tensor_scale + seg, static_cast<hipStream_t>(stream)));
}

attnq_status attnq_quantize_nvfp4_staged(const attnq_theta* theta, const attnq_nvfp4* dst, int32_t seg, void* workspace,
                                         int64_t workspace_bytes, attnq_stream stream) {
  attnq_status st = check_theta(theta);
  if (st != ATTNQ_OK) return st;
  st = check_nvfp4(dst);
  if (st != ATTNQ_OK) return st;
  if (theta->K != dst->K) return ATTNQ_ERR_SHAPE;
  if (seg < 0 || seg >= dst->n_seg) return ATTNQ_ERR_SEGMENT;
  const int32_t start = seg == 0 ? 0 : dst->seg_end[seg - 1];
  if (dst->seg_end[seg] - start != theta->N) return ATTNQ_ERR_SEGMENT;
  const int64_t need = attnq::quantize_staged_workspace_bytes(theta->N, theta->K, theta->r);
  if (need > 0) {
    if (workspace == nullptr) return ATTNQ_ERR_NULL;
    if (workspace_bytes < need) return ATTNQ_ERR_SHAPE;
    if (!aligned(workspace, 256)) return ATTNQ_ERR_ALIGN;
  }
  uint8_t* codes = dst->codes + (size_t)start * (dst->K / 2);
  uint8_t* scales = dst->scales + (size_t)start * (dst->K / 16);
  return from_hip(attnq::launch_quantize_staged(*theta, codes, scales, dst->tensor_scale + seg, workspace,
                                                static_cast<hipStream_t>(stream)));
}

int64_t attnq_quantize_nvfp4_staged_workspace(int32_t N, int32_t K, int32_t r) {
  return attnq::quantize_staged_workspace_bytes(N, K, r);
}

int64_t attnq_quantize_nvfp4_staged_batch_workspace(const attnq_theta* thetas, int32_t count) {
  if (count < 0 || count > ATTNQ_MAX_BATCH || (count > 0 && thetas == nullptr)) return -1;
  return attnq::quantize_staged_batch_workspace_bytes(thetas, count);
}

attnq_status attnq_quantize_nvfp4_staged_batch(const attnq_theta* thetas, const attnq_nvfp4* dsts, const int32_t* segs,
                                               int32_t count, void* workspace, int64_t workspace_bytes,
                                               attnq_stream stream) {
  if (count < 0 || count > ATTNQ_MAX_BATCH) return ATTNQ_ERR_SHAPE;
  if (count == 0) return ATTNQ_OK;
  if (thetas == nullptr || dsts == nullptr || segs == nullptr) return ATTNQ_ERR_NULL;
  uint8_t* codes[ATTNQ_MAX_BATCH];
  uint8_t* scales[ATTNQ_MAX_BATCH];
  float* slots[ATTNQ_MAX_BATCH];
  for (int i = 0; i < count; ++i) {
    const attnq_theta* theta = thetas + i;
    const attnq_nvfp4* dst = dsts + i;
    const int32_t seg = segs[i];
    attnq_status st = check_theta(theta);
    if (st != ATTNQ_OK) return st;
    st = check_nvfp4(dst);
    if (st != ATTNQ_OK) return st;
    if (theta->K != dst->K) return ATTNQ_ERR_SHAPE;
    if (seg < 0 || seg >= dst->n_seg) return ATTNQ_ERR_SEGMENT;
    const int32_t start = seg == 0 ? 0 : dst->seg_end[seg - 1];
    if (dst->seg_end[seg] - start != theta->N) return ATTNQ_ERR_SEGMENT;
    codes[i] = dst->codes + (size_t)start * (dst->K / 2);
    scales[i] = dst->scales + (size_t)start * (dst->K / 16);
    slots[i] = dst->tensor_scale + seg;
    for (int k = 0; k < i; ++k)
      if (slots[k] == slots[i]) return ATTNQ_ERR_SEGMENT;
  }
  const int64_t need = attnq::quantize_staged_batch_workspace_bytes(thetas, count);
  if (need > 0) {
    if (workspace == nullptr) return ATTNQ_ERR_NULL;
    if (workspace_bytes < need) return ATTNQ_ERR_SHAPE;
    if (!aligned(workspace, 256)) return ATTNQ_ERR_ALIGN;
  }
  return from_hip(attnq::launch_quantize_staged_batch(thetas, codes, scales, slots, count, workspace,
                                                      static_cast<hipStream_t>(stream)));
}

attnq_status attnq_gemv_nvfp4(const attnq_nvfp4* W, const uint16_t* x, float* y, attnq_stream stream) {
  attnq_status st = check_nvfp4(W);
  if (st != ATTNQ_OK) return st;
  if (x == nullptr || (y == nullptr && W->N != 0)) return ATTNQ_ERR_NULL;
  if (!aligned(x, 16) || !aligned(y, 4)) return ATTNQ_ERR_ALIGN;
  return from_hip(attnq::launch_gemv_nvfp4(*W, x, y, static_cast<hipStream_t>(stream)));
}

attnq_status attnq_gemv_nvfp4_splitk(const attnq_nvfp4* W, const uint16_t* x, float* y, void* ws, int64_t ws_bytes,
                                     attnq_stream stream) {
  attnq_status st = check_nvfp4(W);
  if (st != ATTNQ_OK) return st;
  if (x == nullptr || (y == nullptr && W->N != 0)) return ATTNQ_ERR_NULL;
  if (!aligned(x, 16) || !aligned(y, 4)) return ATTNQ_ERR_ALIGN;
  const int64_t need = attnq::gemv_nvfp4_splitk_workspace_bytes(W->N, W->K);
  if (need > 0) {
    if (ws == nullptr) return ATTNQ_ERR_NULL;
    if (ws_bytes < need) return ATTNQ_ERR_SHAPE;
    if (!aligned(ws, 256)) return ATTNQ_ERR_ALIGN;
  }
  return from_hip(attnq::launch_gemv_nvfp4_splitk(*W, x, y, ws, static_cast<hipStream_t>(stream)));
}

attnq_status attnq_gemv_nvfp4_splitk_noalloc(const attnq_nvfp4* W, const uint16_t* x, float* y, attnq_stream stream) {
  attnq_status st = check_nvfp4(W);
  if (st != ATTNQ_OK) return st;
  if (x == nullptr || (y == nullptr && W->N != 0)) return ATTNQ_ERR_NULL;
  if (!aligned(x, 16) || !aligned(y, 4)) return ATTNQ_ERR_ALIGN;
  if (attnq::gemv_nvfp4_splitk_workspace_bytes(W->N, W->K) > attnq::gemv_nvfp4_splitk_noalloc_max_bytes())
    return ATTNQ_ERR_SHAPE;
  return from_hip(attnq::launch_gemv_nvfp4_splitk_noalloc(*W, x, y, static_cast<hipStream_t>(stream)));
}

int64_t attnq_gemv_nvfp4_splitk_workspace(int32_t N, int32_t K) {
  if (N < 0 || K <= 0 || K % 32 != 0) return -1;
  return attnq::gemv_nvfp4_splitk_workspace_bytes(N, K);
}

attnq_status attnq_gemv_nvfp4_glu(const attnq_nvfp4* W, const uint16_t* x, int32_t act, uint16_t* h,
                                  attnq_stream stream) {
  attnq_status st = check_nvfp4(W);
  if (st != ATTNQ_OK) return st;
  if (W->n_seg != 2 || W->seg_end[0] * 2 != W->N) return ATTNQ_ERR_SEGMENT;
  if (act != ATTNQ_ACT_GELU_TANH && act != ATTNQ_ACT_SILU && act != ATTNQ_ACT_IDENTITY) return ATTNQ_ERR_SHAPE;
  if (x == nullptr || (h == nullptr && W->N != 0)) return ATTNQ_ERR_NULL;
  if (!aligned(x, 16) || !aligned(h, 2)) return ATTNQ_ERR_ALIGN;
  return from_hip(attnq::launch_gemv_nvfp4_glu(*W, x, act, h, static_cast<hipStream_t>(stream)));
}

attnq_status attnq_gemv_nvfp4_lowrank(const attnq_nvfp4* W0, const uint16_t* s, const uint16_t* U, const uint16_t* V,
                                      int32_t r, const uint16_t* x, float* ws, float* y, attnq_stream stream) {
  attnq_status st = check_nvfp4(W0);
  if (st != ATTNQ_OK) return st;
  if (r < 0 || r > kMaxRank) return ATTNQ_ERR_SHAPE;
  if (x == nullptr || (y == nullptr && W0->N != 0)) return ATTNQ_ERR_NULL;
  if (r > 0 && ((U == nullptr && W0->N != 0) || V == nullptr || ws == nullptr)) return ATTNQ_ERR_NULL;
  if (!aligned(x, 16) || !aligned(y, 4) || !aligned(ws, 4) || !aligned(s, 2) || !aligned(U, 2) || !aligned(V, 16))
    return ATTNQ_ERR_ALIGN;
  return from_hip(attnq::launch_gemv_nvfp4_lowrank(*W0, s, U, V, r, x, ws, y, static_cast<hipStream_t>(stream)));
}

attnq_status attnq_gemv_nvfp4_lowrank_splitk(const attnq_nvfp4* W0, const uint16_t* s, const uint16_t* U,
                                             const uint16_t* V, int32_t r, const uint16_t* x, float* ws,
                                             void* split_ws, int64_t split_ws_bytes, float* y, attnq_stream stream) {
  attnq_status st = check_nvfp4(W0);
  if (st != ATTNQ_OK) return st;
  if (r < 0 || r > kMaxRank) return ATTNQ_ERR_SHAPE;
  if (x == nullptr || (y == nullptr && W0->N != 0)) return ATTNQ_ERR_NULL;
  if (r > 0 && ((U == nullptr && W0->N != 0) || V == nullptr || ws == nullptr)) return ATTNQ_ERR_NULL;
  if (!aligned(x, 16) || !aligned(y, 4) || !aligned(ws, 4) || !aligned(s, 2) || !aligned(U, 2) || !aligned(V, 16))
    return ATTNQ_ERR_ALIGN;
  const int64_t need = attnq::gemv_nvfp4_splitk_workspace_bytes(W0->N, W0->K);
  if (need > 0) {
    if (split_ws == nullptr) return ATTNQ_ERR_NULL;
    if (split_ws_bytes < need) return ATTNQ_ERR_SHAPE;
    if (!aligned(split_ws, 256)) return ATTNQ_ERR_ALIGN;
  }
  return from_hip(attnq::launch_gemv_nvfp4_lowrank_splitk(*W0, s, U, V, r, x, ws, split_ws, y,
                                                          static_cast<hipStream_t>(stream)));
}

int64_t attnq_gemv_nvfp4_lowrank_workspace(int32_t K, int32_t n_seg, int32_t r) {
  if (K <= 0 || K % 32 != 0 || n_seg < 1 || n_seg > ATTNQ_MAX_SEGMENTS || r < 0 || r > kMaxRank) return -1;
  return attnq::lowrank_workspace_floats(K, n_seg, r);
}

attnq_status attnq_gemv_bf16(const uint16_t* W, int32_t N, int32_t K, const uint16_t* x, float* y, attnq_stream stream) {
  if (N < 0 || K <= 0 || K % 32 != 0) return ATTNQ_ERR_SHAPE;
  if (x == nullptr || ((W == nullptr || y == nullptr) && N != 0)) return ATTNQ_ERR_NULL;
  if (!aligned(W, 16) || !aligned(x, 16) || !aligned(y, 4)) return ATTNQ_ERR_ALIGN;
  return from_hip(attnq::launch_gemv_bf16(W, N, K, x, y, static_cast<hipStream_t>(stream)));
}

attnq_status attnq_gemm_nvfp4_small_m(const attnq_nvfp4* W, const uint16_t* X, int32_t M, int32_t ldx, float* Y,
                                      int32_t ldy, attnq_stream stream) {
  attnq_status st = check_nvfp4(W);
  if (st != ATTNQ_OK) return st;
  if (M < 0 || M > kMaxM || ldx < W->K || ldx % 8 != 0 || ldy < W->N) return ATTNQ_ERR_SHAPE;
  // X is addressed with 32-bit byte offsets inside the kernels: its extent must stay below 2^30 elements
  if (M > 0 && (int64_t)(M - 1) * ldx + W->K >= (int64_t{1} << 30)) return ATTNQ_ERR_SHAPE;
  if ((X == nullptr || Y == nullptr) && M != 0 && W->N != 0) return ATTNQ_ERR_NULL;
  if (!aligned(X, 16) || !aligned(Y, 4)) return ATTNQ_ERR_ALIGN;
  return from_hip(attnq::launch_gemm_nvfp4_small_m(*W, X, M, ldx, Y, ldy, static_cast<hipStream_t>(stream)));
}

attnq_status attnq_gemm_nvfp4_small_m_splitk(const attnq_nvfp4* W, const uint16_t* X, int32_t M, int32_t ldx, float* Y,
                                             int32_t ldy, void* ws, int64_t ws_bytes, attnq_stream stream) {
  attnq_status st = check_nvfp4(W);
  if (st != ATTNQ_OK) return st;
  if (M < 0 || M > kMaxM || ldx < W->K || ldx % 8 != 0 || ldy < W->N) return ATTNQ_ERR_SHAPE;
  if (M > 0 && (int64_t)(M - 1) * ldx + W->K >= (int64_t{1} << 30)) return ATTNQ_ERR_SHAPE;
  if ((X == nullptr || Y == nullptr) && M != 0 && W->N != 0) return ATTNQ_ERR_NULL;
  if (!aligned(X, 16) || !aligned(Y, 4)) return ATTNQ_ERR_ALIGN;
  const int64_t need = attnq::gemm_small_m_splitk_workspace_bytes(W->N, W->K, M);
  if (need > 0) {
    if (ws == nullptr) return ATTNQ_ERR_NULL;
    if (ws_bytes < need) return ATTNQ_ERR_SHAPE;
    if (!aligned(ws, 256)) return ATTNQ_ERR_ALIGN;
  }
  return from_hip(attnq::launch_gemm_nvfp4_small_m_splitk(*W, X, M, ldx, Y, ldy, ws, static_cast<hipStream_t>(stream)));
}

int64_t attnq_gemm_nvfp4_small_m_splitk_workspace(int32_t N, int32_t K, int32_t M) {
  if (N < 0 || K <= 0 || K % 32 != 0 || M < 0 || M > kMaxM) return -1;
  return attnq::gemm_small_m_splitk_workspace_bytes(N, K, M);
}

attnq_status attnq_read_ceiling(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes, uint32_t* sink,
                                attnq_stream stream) {
  if (a_bytes < 0 || b_bytes < 0 || a_bytes % 16 != 0 || b_bytes % 16 != 0) return ATTNQ_ERR_SHAPE;
  if (a_bytes + b_bytes >= (int64_t{63} << 30)) return ATTNQ_ERR_SHAPE;   // 32-bit piece indices
  if ((a == nullptr && a_bytes > 0) || (b == nullptr && b_bytes > 0) || sink == nullptr) return ATTNQ_ERR_NULL;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(sink, 4)) return ATTNQ_ERR_ALIGN;
  return from_hip(attnq::launch_read_ceiling(a, a_bytes, b, b_bytes, sink, static_cast<hipStream_t>(stream)));
}

const char* attnq_status_string(attnq_status status) {
  switch (status) {
    case ATTNQ_OK: return "ATTNQ_OK";
    case ATTNQ_ERR_NULL: return "ATTNQ_ERR_NULL: a required pointer is NULL";
    case ATTNQ_ERR_SHAPE: return "ATTNQ_ERR_SHAPE: a size is out of range";
    case ATTNQ_ERR_ALIGN: return "ATTNQ_ERR_ALIGN: a device pointer is misaligned";
    case ATTNQ_ERR_SEGMENT: return "ATTNQ_ERR_SEGMENT: segment table or index inconsistent";
    case ATTNQ_ERR_LAYOUT: return "ATTNQ_ERR_LAYOUT: unknown packed-weight layout";
    case ATTNQ_ERR_HIP: return "ATTNQ_ERR_HIP: a kernel launch failed";
  }
  return "attnq: unknown status";
}

}  // extern "C"
