// Small-M NVFP4 product Y = X * W^T for M <= 16 token rows: speculative verification of
// gamma = 3 drafted tokens plus one ("Throughput", "Speculative decoding") and batch 8.
//
// This kernel keeps the GEMV's streaming layout (a lane owns a 16-byte code chunk of R rows);
// each chunk is decoded once to bf16 and reused for every token row.
#include "attnq_device.h"
#include "launch.h"

namespace attnq {

namespace {

template <int MT>
__global__ __launch_bounds__(256) void k_gemm_small_m(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                                      const float* __restrict__ tensor_scale, SegTable segs,
                                                      const uint16_t* __restrict__ X, int M, int ldx,
                                                      float* __restrict__ Y, int ldy, int N, int K) {
  constexpr int R = 2;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row0 = (blockIdx.x * 4 + wave) * R;
  const int cpr = K >> 5;
  const size_t code_pitch = (size_t)K >> 1;
  const size_t scale_pitch = (size_t)K >> 4;
  float acc[MT][R];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[m][r] = 0.0f;

  for (int c = lane; c < cpr; c += 64) {
    uint32_t w[R][16];
    float s0[R], s1[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = min(row0 + r, N - 1);
      const u32x4 cv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(codes + row * code_pitch) + c);
      const uint32_t sv = *reinterpret_cast<const uint16_t*>(scales + row * scale_pitch + 2 * c);
      s0[r] = __builtin_amdgcn_cvt_f32_fp8((int)sv, 0);
      s1[r] = __builtin_amdgcn_cvt_f32_fp8((int)sv, 1);
      const uint32_t cw[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        w[r][4 * j + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[j], 1.0f, 0));
        w[r][4 * j + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[j], 1.0f, 1));
        w[r][4 * j + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[j], 1.0f, 2));
        w[r][4 * j + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[j], 1.0f, 3));
      }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m < M) {
        const u32x4* xp = reinterpret_cast<const u32x4*>(X + (size_t)m * ldx + (size_t)c * kChunkElems);
        const u32x4 x0 = xp[0], x1 = xp[1], x2 = xp[2], x3 = xp[3];
        const uint32_t xw[16] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,
                                 x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
          for (int j = 0; j < 8; ++j)
            p0 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w[r][j]), as_bf16x2(xw[j]), p0, false);
#pragma unroll
          for (int j = 8; j < 16; ++j)
            p1 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w[r][j]), as_bf16x2(xw[j]), p1, false);
          acc[m][r] = __builtin_fmaf(p0, s0[r], acc[m][r]);
          acc[m][r] = __builtin_fmaf(p1, s1[r], acc[m][r]);
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    if (m < M) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float v = wave_sum(acc[m][r]);
        const int row = row0 + r;
        if (lane == 0 && row < N) Y[(size_t)m * ldy + row] = v * tensor_scale[segment_of(segs, row)];
      }
    }
  }
}

template <int MT>
void launch_mt(const attnq_nvfp4& W, const uint16_t* X, int M, int ldx, float* Y, int ldy, hipStream_t stream) {
  SegTable t;
  t.n_seg = W.n_seg;
  for (int i = 0; i < ATTNQ_MAX_SEGMENTS; ++i) t.end[i] = (i < W.n_seg) ? W.seg_end[i] : W.N;
  const unsigned grid = (unsigned)((W.N + 7) / 8);
  k_gemm_small_m<MT><<<grid, 256, 0, stream>>>(W.codes, W.scales, W.tensor_scale, t, X, M, ldx, Y, ldy, W.N, W.K);
}

}  // namespace

hipError_t launch_gemm_nvfp4_small_m(const attnq_nvfp4& W, const uint16_t* X, int M, int ldx, float* Y, int ldy,
                                     hipStream_t stream) {
  if (W.N == 0 || M == 0) return hipSuccess;
  if (M <= 4)
    launch_mt<4>(W, X, M, ldx, Y, ldy, stream);
  else if (M <= 8)
    launch_mt<8>(W, X, M, ldx, Y, ldy, stream);
  else
    launch_mt<16>(W, X, M, ldx, Y, ldy, stream);
  return hipGetLastError();
}

}  // namespace attnq
