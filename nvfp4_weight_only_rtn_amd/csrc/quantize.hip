// Load path: reconstruction W_eff = s*W0 + U*V^T and NVFP4 round-to-nearest quantization.
//
// Reconstruction: AttnQuant landing page, "How it works" (theta bundle rebuilt once at load);
// weightless "GPU and cache acceleration", "Precompute-outside". Quantization: "GPU
// acceleration", "NVFP4 quantization" (packed uint8 plus float8 block scales, at load);
// landing page "Results" (round-to-nearest, no calibration); "Throughput", "What quantization
// actually saves" (an E4M3 scale byte for each block of 16 elements).
//
// Rank 0 (passthrough or row scale only): one thread owns one 16-element block of a row, rebuilds
// it in registers, rounds it to bf16 and then either folds |w| into the segment amax or emits 8
// code bytes and one scale byte. The fused path rebuilds twice (amax pass, then quantize pass)
// instead of staging W_eff in HBM: 2 + 2 + 0.5625 B of traffic per element.
//
// Rank r > 0: a workgroup rebuilds a 64-row x 256-column tile. V for the tile's columns and U for
// its rows are staged in LDS as fp32 [k][column] and [k][row], 32 values of k at a time, and each
// thread keeps a 4-row x 16-column block of fp32 accumulators, so every V value read from LDS
// feeds four rows. The accumulation order (k ascending from +0, then s*W0 + acc) is the same in
// both paths.
#include "attnq_device.h"
#include "launch.h"

namespace attnq {

namespace {

struct Theta {
  const uint16_t* W0;
  const uint16_t* s;
  const uint16_t* U;
  const uint16_t* V;
  int N, K, r;
};

// Two fp32 values -> two bf16 (round to nearest even, NaN kept quiet), packed low = first. The
// gfx950 converter (v_cvt_pk_bf16_f32) matches the bit-level rule of f32_to_bf16_bits exactly.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  const bf16x2v p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}
__device__ __forceinline__ float bf16_lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t p) { return __uint_as_float(p & 0xFFFF0000u); }

// Two fp32 quotients -> two E2M1 codes in byte `j` of `acc` (even element in the low nibble):
// v_cvt_scalef32_pk_fp4_f32 with scale 1 rounds to the nearest grid value with ties to the even
// code, saturates at 6 and copies the sign, which is e2m1_magnitude plus the sign bit for every
// non-NaN input.
__device__ __forceinline__ uint32_t cvt_fp4_pair(uint32_t acc, float a, float b, int j) {
  switch (j) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, a, b, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, a, b, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, a, b, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, a, b, 1.0f, 3);
  }
}

// Round a rebuilt 16-element block (eight packed bf16 pairs, element 2i in the low half of
// wp[i]) to NVFP4 with the segment's amax bits: 8 packed code bytes (even element in the low
// nibble) and one E4M3 scale code.
//
// The element quotient q = fl32(w / d) uses one correctly rounded reciprocal y = 1/d per block:
// q0 = w*y, r = fma(-q0, d, w) (exact), q = fma(r, y, q0) is the correctly rounded quotient when
// d and y are normal (Markstein's theorem); its sign is copied from w so that -0 stays -0. A block whose d is zero or subnormal falls back to
// the exact division and the software rounding rule (e2m1_magnitude), as does 0/0 there.
__device__ __forceinline__ void quantize_block(const uint32_t wp[kBlock / 2], uint32_t ts_bits, uint32_t packed[2],
                                               uint32_t& scale_code) {
  const float ts = __uint_as_float(ts_bits);
  const float six_ts = 6.0f * ts;
  uint32_t bmax = 0;
#pragma unroll
  for (int i = 0; i < kBlock / 2; ++i) bmax = max(bmax, max(wp[i] & 0x7FFFu, (wp[i] >> 16) & 0x7FFFu));
  const float bamax = bf16_bits_to_f32(bmax);
  const float sb = (ts_bits == 0u) ? 0.0f : bamax / six_ts;     // ts == 0 exactly when amax == 0
  const uint32_t S = e4m3_encode_nonneg(sb);
  const float d = e4m3_to_f32(S) * ts;
  scale_code = S;
  float w[kBlock];
#pragma unroll
  for (int i = 0; i < kBlock / 2; ++i) {
    w[2 * i] = bf16_lo(wp[i]);
    w[2 * i + 1] = bf16_hi(wp[i]);
  }
  packed[0] = 0u;
  packed[1] = 0u;
  if (S != 0u && !(d >= 0x1p-126f)) {
#pragma unroll
    for (int i = 0; i < kBlock; ++i) {
      const uint32_t sign = (__float_as_uint(w[i]) >> 28) & 8u;
      packed[i >> 3] |= (sign | e2m1_magnitude(__builtin_fabsf(w[i] / d))) << (4 * (i & 7));
    }
    return;
  }
  float q[kBlock];
  if (S == 0u) {
#pragma unroll
    for (int i = 0; i < kBlock; ++i) q[i] = w[i] * 0.0f;          // magnitude 0, sign of w
  } else {
    const float y = 1.0f / d;
#pragma unroll
    for (int i = 0; i < kBlock; ++i) {
      const float q0 = w[i] * y;
      // the correction rounds -0 + +0 to +0: the quotient takes the sign of w explicitly
      q[i] = __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-q0, d, w[i]), y, q0), w[i]);
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    packed[0] = cvt_fp4_pair(packed[0], q[2 * j], q[2 * j + 1], j);
    packed[1] = cvt_fp4_pair(packed[1], q[8 + 2 * j], q[8 + 2 * j + 1], j);
  }
}

// ---------------------------------------------------------------------------------- rank 0
// Rebuild 16 consecutive elements [col, col+16) of row `row` as eight packed bf16 pairs (r == 0).
__device__ __forceinline__ void rebuild_block_r0(const Theta& t, int row, int col, uint32_t wp[kBlock / 2]) {
  const u32x4* src = reinterpret_cast<const u32x4*>(t.W0 + (size_t)row * t.K + col);
  const u32x4 a = __builtin_nontemporal_load(src);
  const u32x4 b = __builtin_nontemporal_load(src + 1);
  const uint32_t w0[kBlock / 2] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  if (t.s == nullptr) {                             // passthrough: W_eff = W0 bit for bit
#pragma unroll
    for (int i = 0; i < kBlock / 2; ++i) wp[i] = w0[i];
    return;
  }
  const float si = bf16_bits_to_f32(t.s[row]);
#pragma unroll
  for (int i = 0; i < kBlock / 2; ++i)              // bf16 x bf16 products are exact in fp32
    wp[i] = pack_bf16(si * bf16_lo(w0[i]), si * bf16_hi(w0[i]));
}

// Fold the |w| bit patterns of eight packed bf16 pairs into a running max (as fp32 bit patterns;
// NaN patterns sort above +inf).
__device__ __forceinline__ uint32_t amax_bits_of(const uint32_t wp[kBlock / 2], uint32_t m) {
#pragma unroll
  for (int i = 0; i < kBlock / 2; ++i) m = max(m, max((wp[i] << 16) & 0x7FFF0000u, wp[i] & 0x7FFF0000u));
  return m;
}

__global__ __launch_bounds__(256) void k_reconstruct_r0(Theta t, uint16_t* __restrict__ out, int64_t nblocks) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  const int bpr = t.K / kBlock;
  const int row = (int)(b / bpr), col = (int)(b % bpr) * kBlock;
  uint32_t wp[kBlock / 2];
  rebuild_block_r0(t, row, col, wp);
  u32x4* dst = reinterpret_cast<u32x4*>(out + (size_t)row * t.K + col);
  dst[0] = u32x4{wp[0], wp[1], wp[2], wp[3]};
  dst[1] = u32x4{wp[4], wp[5], wp[6], wp[7]};
}

__global__ void k_zero_slot(uint32_t* slot) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *slot = 0u;
}

// Workgroup max of per-thread |w| bit patterns, turned into the workgroup's tensor scale
// fl32(amax / 2688) (NaN for a non-finite amax) and folded into the segment slot with atomicMax
// on its bit pattern. A correctly rounded division by a positive constant is monotone, so the
// largest workgroup scale is the segment's; the max of bit patterns is order-free, hence
// deterministic, and NaN sorts above every finite scale. The slot ends holding the tensor scale.
__device__ __forceinline__ void fold_tensor_scale(uint32_t m, uint32_t* slot) {
  __shared__ uint32_t red[4];
  m = wave_max_u32(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = max(max(red[0], red[1]), max(red[2], red[3]));
    if (m) atomicMax(slot, __float_as_uint(tensor_scale_from_amax_bits(m)));
  }
}

__global__ __launch_bounds__(256) void k_amax_r0(Theta t, uint32_t* slot, int64_t nblocks) {
  uint32_t m = 0;
  const int bpr = t.K / kBlock;
  for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < nblocks; b += (int64_t)gridDim.x * 256) {
    const int row = (int)(b / bpr), col = (int)(b % bpr) * kBlock;
    uint32_t wp[kBlock / 2];
    rebuild_block_r0(t, row, col, wp);
    m = amax_bits_of(wp, m);
  }
  fold_tensor_scale(m, slot);
}

__global__ __launch_bounds__(256) void k_quantize_r0(Theta t, const uint32_t* __restrict__ slot, uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales, int64_t nblocks) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  const int bpr = t.K / kBlock;
  const int row = (int)(b / bpr), cb = (int)(b % bpr);
  const uint32_t ts_bits = *slot;
  u32x2* cdst = reinterpret_cast<u32x2*>(codes + (size_t)row * (t.K / 2) + cb * (kBlock / 2));
  uint8_t* sdst = scales + (size_t)row * bpr + cb;
  if (ts_bits >= 0x7F800000u) {                     // non-finite segment (ts NaN): NaN scales, zero codes
    *cdst = u32x2{0u, 0u};
    *sdst = 0x7F;
    return;
  }
  uint32_t wp[kBlock / 2];
  rebuild_block_r0(t, row, cb * kBlock, wp);
  uint32_t packed[2], S;
  quantize_block(wp, ts_bits, packed, S);
  *cdst = u32x2{packed[0], packed[1]};
  *sdst = (uint8_t)S;
}

// ---------------------------------------------------------------------------------- rank > 0
constexpr int kTileRows = 64;
constexpr int kTileCols = 256;
constexpr int kRowsPerThread = 4;   // 256 threads = 16 column blocks x 16 row groups of 4 rows
constexpr int kRankChunk = 32;      // values of k staged in LDS at a time
// LDS row strides (floats) of the staged V [k][column] and U [k][row] tiles: padded by 4 so the
// transposing writes spread over the banks while rows stay 16-byte aligned for the f32x4 reads.
constexpr int kVStride = kTileCols + 4;
constexpr int kUStride = kTileRows + 4;

enum LowRankPass { kPassAmax = 0, kPassQuantize = 1, kPassReconstruct = 2 };

size_t lowrank_lds_bytes(int r) { return (size_t)min(r, kRankChunk) * (kVStride + kUStride) * 4; }

// e / n for 0 <= e < 2^16 and 1 <= n <= 32: the reciprocal product lands at least 1/64 away from
// the next integer, far beyond its rounding error.
__device__ __forceinline__ int div_small(int e, float inv_n) { return (int)(((float)e + 0.5f) * inv_n); }

// Stage columns k0 .. k0+kn-1 of the tile's V rows (col0 .. col0+255, zero past K) and U rows
// (row0 .. row0+63, zero past N) into LDS as fp32 vt[k * kVStride + column] and
// ut[k * kUStride + row]. The two are one flat element space (V first); consecutive threads read
// consecutive elements, and each thread issues up to kStageBatch loads before any LDS write, so a
// rank chunk of up to 16 is staged in one round trip. Only the loaded values stay live across
// the batch; each element's place is worked out again when it is written.
constexpr int kStageBatch = 20;

struct StageElem {
  const uint16_t* src;
  int index;        // element of src, clamped into the matrix
  int slot;         // LDS float index relative to vt
  bool inside;      // false: the row is past the matrix, the slot takes 0
};

__device__ __forceinline__ StageElem stage_elem(const Theta& t, int row0, int col0, int k0, int kn, float inv_kn,
                                                int nv, int e, int u_off) {
  const bool is_v = e < nv;
  const int f = is_v ? e : e - nv;
  const int row = div_small(f, inv_kn), k = f - row * kn;
  const int base = is_v ? col0 : row0, limit = is_v ? t.K : t.N;
  StageElem s;
  s.src = is_v ? t.V : t.U;
  s.index = min(base + row, limit - 1) * t.r + k0 + k;
  s.slot = is_v ? k * kVStride + row : u_off + k * kUStride + row;
  s.inside = base + row < limit;
  return s;
}

__device__ __forceinline__ void stage_uv(const Theta& t, int row0, int col0, int k0, int kn, float inv_kn, float* vt,
                                         float* ut) {
  const int nv = kTileCols * kn, total = (kTileCols + kTileRows) * kn;
  const int u_off = (int)(ut - vt);
  for (int e0 = 0; e0 < total; e0 += kStageBatch * 256) {
    uint16_t v[kStageBatch];
#pragma unroll
    for (int j = 0; j < kStageBatch; ++j) {       // clamped, branch-free loads, all issued first
      const StageElem s = stage_elem(t, row0, col0, k0, kn, inv_kn, nv, min(e0 + j * 256 + (int)threadIdx.x, total - 1), u_off);
      v[j] = s.src[s.index];
    }
#pragma unroll
    for (int j = 0; j < kStageBatch; ++j) {
      const int e = e0 + j * 256 + (int)threadIdx.x;
      if (e < total) {
        const StageElem s = stage_elem(t, row0, col0, k0, kn, inv_kn, nv, e, u_off);
        vt[s.slot] = s.inside ? bf16_bits_to_f32(v[j]) : 0.0f;
      }
    }
  }
}

// One thread rebuilds rows row0 + 4*rg .. +3, columns col .. col+15 of a 64 x 256 tile.
template <int PASS>
__global__ __launch_bounds__(256) void k_lowrank_tile(Theta t, uint32_t* slot, uint8_t* __restrict__ codes,
                                                      uint8_t* __restrict__ scales, uint16_t* __restrict__ out,
                                                      int tiles_c) {
  extern __shared__ float lds[];
  const int r = t.r;
  const int rc = min(r, kRankChunk);
  float* vt = lds;                              // [rc][kVStride]
  float* ut = lds + (size_t)rc * kVStride;      // [rc][kUStride]
  const int tile_r = blockIdx.x / tiles_c, tile_c = blockIdx.x % tiles_c;
  const int row0 = tile_r * kTileRows, col0 = tile_c * kTileCols;

  uint32_t ts_bits = 0;
  if (PASS == kPassQuantize) {
    ts_bits = *slot;
    if (ts_bits >= 0x7F800000u) {                 // non-finite segment (ts NaN): NaN scales, zero codes
      const int cb = threadIdx.x & 15, rg = threadIdx.x >> 4;
      const int col = col0 + cb * kBlock;
      for (int rr = 0; rr < kRowsPerThread; ++rr) {
        const int row = row0 + rg * kRowsPerThread + rr;
        if (row < t.N && col < t.K) {
          *reinterpret_cast<u32x2*>(codes + (size_t)row * (t.K / 2) + col / 2) = u32x2{0u, 0u};
          scales[(size_t)row * (t.K / kBlock) + col / kBlock] = 0x7F;
        }
      }
      return;
    }
  }

  const int cb = threadIdx.x & 15, rg = threadIdx.x >> 4;
  const int col = col0 + cb * kBlock;
  const bool col_ok = col < t.K;                 // K % 16 == 0, so the whole block is inside
  float acc[kRowsPerThread][kBlock];
#pragma unroll
  for (int rr = 0; rr < kRowsPerThread; ++rr)
#pragma unroll
    for (int i = 0; i < kBlock; ++i) acc[rr][i] = 0.0f;
  for (int k0 = 0; k0 < r; k0 += kRankChunk) {
    const int kn = min(kRankChunk, r - k0);
    if (k0 > 0) __syncthreads();                 // previous chunk fully consumed
    // stage V (tile columns) and U (tile rows) for k0 .. k0+kn-1, transposed to [k][.]; zero
    // outside the matrix
    stage_uv(t, row0, col0, k0, kn, 1.0f / (float)kn, vt, ut);
    __syncthreads();
    for (int k = 0; k < kn; ++k) {               // k ascending: one fp32 rounding per step
      const f32x4* vp = reinterpret_cast<const f32x4*>(vt + k * kVStride + cb * kBlock);
      const f32x4 v0 = vp[0], v1 = vp[1], v2 = vp[2], v3 = vp[3];
      const float v[kBlock] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w,
                               v2.x, v2.y, v2.z, v2.w, v3.x, v3.y, v3.z, v3.w};
      const f32x4 up = *reinterpret_cast<const f32x4*>(ut + k * kUStride + rg * kRowsPerThread);
      const float u[kRowsPerThread] = {up.x, up.y, up.z, up.w};
#pragma unroll
      for (int rr = 0; rr < kRowsPerThread; ++rr)
#pragma unroll
        for (int i = 0; i < kBlock; ++i) acc[rr][i] = __builtin_fmaf(u[rr], v[i], acc[rr][i]);
    }
  }

  int rows[kRowsPerThread];
  u32x4 w0a[kRowsPerThread], w0b[kRowsPerThread];
  float si[kRowsPerThread];
#pragma unroll
  for (int rr = 0; rr < kRowsPerThread; ++rr) {
    rows[rr] = row0 + rg * kRowsPerThread + rr;
    const int row = min(rows[rr], t.N - 1);      // clamped load; results of rows past N are dropped
    const int cc = col_ok ? col : 0;
    const u32x4* src = reinterpret_cast<const u32x4*>(t.W0 + (size_t)row * t.K + cc);
    w0a[rr] = __builtin_nontemporal_load(src);
    w0b[rr] = __builtin_nontemporal_load(src + 1);
    si[rr] = t.s ? bf16_bits_to_f32(t.s[row]) : 1.0f;
  }
  uint32_t m = 0;
#pragma unroll
  for (int rr = 0; rr < kRowsPerThread; ++rr) {
    const uint32_t ww[8] = {w0a[rr].x, w0a[rr].y, w0a[rr].z, w0a[rr].w, w0b[rr].x, w0b[rr].y, w0b[rr].z, w0b[rr].w};
    uint32_t wp[kBlock / 2];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      wp[i] = pack_bf16(__builtin_fmaf(si[rr], bf16_lo(ww[i]), acc[rr][2 * i]),
                        __builtin_fmaf(si[rr], bf16_hi(ww[i]), acc[rr][2 * i + 1]));
    const bool ok = col_ok && rows[rr] < t.N;
    if (PASS == kPassAmax) {
      if (ok) m = amax_bits_of(wp, m);
    } else if (PASS == kPassQuantize) {
      if (ok) {
        uint32_t packed[2], S;
        quantize_block(wp, ts_bits, packed, S);
        *reinterpret_cast<u32x2*>(codes + (size_t)rows[rr] * (t.K / 2) + col / 2) = u32x2{packed[0], packed[1]};
        scales[(size_t)rows[rr] * (t.K / kBlock) + col / kBlock] = (uint8_t)S;
      }
    } else {
      if (ok) {
        u32x4* dst = reinterpret_cast<u32x4*>(out + (size_t)rows[rr] * t.K + col);
        dst[0] = u32x4{wp[0], wp[1], wp[2], wp[3]};
        dst[1] = u32x4{wp[4], wp[5], wp[6], wp[7]};
      }
    }
  }
  if (PASS == kPassAmax) fold_tensor_scale(m, slot);
}

Theta to_theta(const attnq_theta& t) { return Theta{t.W0, t.s, t.U, t.V, t.N, t.K, t.r}; }

template <int PASS>
void launch_lowrank(const Theta& t, uint32_t* slot, uint8_t* codes, uint8_t* scales, uint16_t* out, hipStream_t stream) {
  const int tiles_r = (t.N + kTileRows - 1) / kTileRows;
  const int tiles_c = (t.K + kTileCols - 1) / kTileCols;
  k_lowrank_tile<PASS><<<(unsigned)tiles_r * tiles_c, 256, lowrank_lds_bytes(t.r), stream>>>(t, slot, codes, scales, out,
                                                                                           tiles_c);
}

}  // namespace

hipError_t launch_reconstruct(const attnq_theta& th, uint16_t* out, hipStream_t stream) {
  const Theta t = to_theta(th);
  const int64_t nblocks = (int64_t)th.N * (th.K / kBlock);
  if (nblocks == 0) return hipSuccess;
  if (t.r == 0)
    k_reconstruct_r0<<<(unsigned)((nblocks + 255) / 256), 256, 0, stream>>>(t, out, nblocks);
  else
    launch_lowrank<kPassReconstruct>(t, nullptr, nullptr, nullptr, out, stream);
  return hipGetLastError();
}

hipError_t launch_quantize(const attnq_theta& th, uint8_t* codes, uint8_t* scales, float* tensor_scale,
                           hipStream_t stream) {
  const Theta t = to_theta(th);
  const int64_t nblocks = (int64_t)th.N * (th.K / kBlock);
  uint32_t* slot = reinterpret_cast<uint32_t*>(tensor_scale);
  k_zero_slot<<<1, 64, 0, stream>>>(slot);
  if (nblocks > 0) {
    if (t.r == 0) {
      const int64_t want = (nblocks + 255) / 256;
      const unsigned amax_grid = (unsigned)(want < 4096 ? want : 4096);
      k_amax_r0<<<amax_grid, 256, 0, stream>>>(t, slot, nblocks);
      k_quantize_r0<<<(unsigned)want, 256, 0, stream>>>(t, slot, codes, scales, nblocks);
    } else {
      launch_lowrank<kPassAmax>(t, slot, nullptr, nullptr, nullptr, stream);
      launch_lowrank<kPassQuantize>(t, slot, codes, scales, nullptr, stream);
    }
  }
  return hipGetLastError();
}

}  // namespace attnq
