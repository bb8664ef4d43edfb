// Device helpers shared by the attnq HIP kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/attnq.h"

namespace attnq {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 16;          // elements per E4M3 block scale
constexpr int kChunkElems = 32;     // one 16-byte code chunk = 32 fp4 = two blocks
constexpr float kTsDivisor = 2688.0f;   // E2M1 max (6) * E4M3 max (448)

// Row segments of a fused weight, passed by value to kernels.
struct SegTable {
  int32_t n_seg;
  int32_t end[ATTNQ_MAX_SEGMENTS];
};

__device__ __forceinline__ int segment_of(const SegTable& t, int row) {
  int s = 0;
#pragma unroll
  for (int i = 0; i < ATTNQ_MAX_SEGMENTS - 1; ++i) s += (i < t.n_seg - 1 && row >= t.end[i]) ? 1 : 0;
  return s;
}

// Reinterpret a dword as two bf16. Always pass a plain value: clang's __builtin_bit_cast on an
// ext-vector element expression (v.y) reads from the start of the vector instead.
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even; NaN becomes a quiet NaN with the same top bits.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Non-negative fp32 -> E4M3FN code: nearest value, ties to the even code, saturating to 448.
// Integer formulation: keep 3 mantissa bits of a normal and round on the 20 dropped ones;
// below 2^-6 the E4M3 grid is uniform with step 2^-9, so round x * 512 to an integer.
__device__ __forceinline__ uint32_t e4m3_encode_nonneg(float x) {
  if (!(x == x)) return 0x7Fu;
  if (x >= 448.0f) return 0x7Eu;
  uint32_t b = __float_as_uint(x);
  int e = (int)(b >> 23) - 127;
  if (e < -6) return (uint32_t)__builtin_rintf(x * 512.0f);   // exact scaling, rint is RNE
  uint32_t mant = b & 0x7FFFFFu;
  uint32_t keep = mant >> 20, rest = mant & 0xFFFFFu;
  uint32_t code = ((uint32_t)(e + 7) << 3) | keep;
  if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) code += 1u;   // carry may bump the exponent
  return code;
}

// |q| -> E2M1 magnitude index (grid 0 .5 1 1.5 2 3 4 6): count the rounding boundaries passed.
// Boundaries at 0.25, 1.25, 2.5, 5 resolve ties downward (to the even index), those at 0.75,
// 1.75, 3.5 upward (also to the even index). NaN passes none and encodes as 0.
__device__ __forceinline__ uint32_t e2m1_magnitude(float a) {
  return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) + (uint32_t)(a >= 1.75f) +
         (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
}

// E4M3FN code -> fp32 via the gfx950 OCP fp8 converter (exact for every code).
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) { return __builtin_amdgcn_cvt_f32_fp8((int)code, 0); }

// Tensor scale from the amax bit pattern (identical expression wherever it is needed).
__device__ __forceinline__ float tensor_scale_from_amax_bits(uint32_t bits) {
  if (bits >= 0x7F800000u) return __uint_as_float(0x7FC00000u);
  return __uint_as_float(bits) / kTsDivisor;
}

// v from the lane CTRL selects (DPP), 0 where the row mask excludes a row or the source lane
// does not exist
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false));
}

// Sums over the 64 lanes of a wave of n values at once; every lane receives the totals. Inside
// each row of 16 lanes, shifts by 1, 2, 4 and 8 leave the row's sum in its last lane;
// row_bcast:15 adds row 0's sum into row 1 and row 2's into row 3, and row_bcast:31 adds lane
// 31's into rows 2 and 3, so lane 63 ends with the total, which is read into a scalar register
// (no LDS round trip). The values advance step by step together, so that independent DPP
// operations fill each other's wait states. All 64 lanes must be active.
template <int n>
__device__ __forceinline__ void wave_sums(float* v) {
#pragma unroll
  for (int i = 0; i < n; ++i) v[i] += dpp_f32<0x111, 0xF>(v[i]);
#pragma unroll
  for (int i = 0; i < n; ++i) v[i] += dpp_f32<0x112, 0xF>(v[i]);
#pragma unroll
  for (int i = 0; i < n; ++i) v[i] += dpp_f32<0x114, 0xF>(v[i]);
#pragma unroll
  for (int i = 0; i < n; ++i) v[i] += dpp_f32<0x118, 0xF>(v[i]);
#pragma unroll
  for (int i = 0; i < n; ++i) v[i] += dpp_f32<0x142, 0xA>(v[i]);
#pragma unroll
  for (int i = 0; i < n; ++i) v[i] += dpp_f32<0x143, 0xC>(v[i]);
#pragma unroll
  for (int i = 0; i < n; ++i) v[i] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v[i]), 63));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, true));
  v = max(v, (uint32_t)__shfl_xor((int)v, 16));
  v = max(v, (uint32_t)__shfl_xor((int)v, 32));
  return v;
}

}  // namespace attnq
