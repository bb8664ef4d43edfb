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
#include <atomic>

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

// Round a rebuilt 16-element block to NVFP4: w holds the block's bf16 values as fp32 and bamax
// their largest magnitude; ts_bits is the segment's tensor scale. Emits 8 packed code bytes (even
// element in the low nibble) and one E4M3 scale code.
//
// The element quotient q = fl32(w / d) uses one correctly rounded reciprocal y = 1/d per block:
// q0 = w*y, r = fma(-q0, d, w) (exact), q = fma(r, y, q0) is the correctly rounded quotient when
// d and y are normal (Markstein's theorem). The correction turns -0 into +0; NEG_ZERO copies the
// sign of w back, which only a block that can hold -0 needs. A block whose d is zero or subnormal
// falls back to the exact division and the software rounding rule (e2m1_magnitude), as does 0/0
// there.
template <bool NEG_ZERO>
__device__ __forceinline__ void quantize_values(const float w[kBlock], float bamax, uint32_t ts_bits, uint32_t packed[2],
                                                uint32_t& scale_code) {
  const float ts = __uint_as_float(ts_bits);
  const float six_ts = 6.0f * ts;
  const float sb = (ts_bits == 0u) ? 0.0f : bamax / six_ts;     // ts == 0 exactly when amax == 0
  const uint32_t S = e4m3_encode_nonneg(sb);
  const float d = e4m3_to_f32(S) * ts;
  scale_code = S;
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
      const float qc = __builtin_fmaf(__builtin_fmaf(-q0, d, w[i]), y, q0);
      q[i] = NEG_ZERO ? __builtin_copysignf(qc, w[i]) : qc;
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    packed[0] = cvt_fp4_pair(packed[0], q[2 * j], q[2 * j + 1], j);
    packed[1] = cvt_fp4_pair(packed[1], q[8 + 2 * j], q[8 + 2 * j + 1], j);
  }
}

// The same from eight packed bf16 pairs (element 2i in the low half of wp[i]); the block amax is
// taken on the bf16 bit patterns.
__device__ __forceinline__ void quantize_block(const uint32_t wp[kBlock / 2], uint32_t ts_bits, uint32_t packed[2],
                                               uint32_t& scale_code) {
  uint32_t bmax = 0;
#pragma unroll
  for (int i = 0; i < kBlock / 2; ++i) bmax = max(bmax, max(wp[i] & 0x7FFFu, (wp[i] >> 16) & 0x7FFFu));
  float w[kBlock];
#pragma unroll
  for (int i = 0; i < kBlock / 2; ++i) {
    w[2 * i] = bf16_lo(wp[i]);
    w[2 * i + 1] = bf16_hi(wp[i]);
  }
  quantize_values<true>(w, bf16_bits_to_f32(bmax), ts_bits, packed, scale_code);
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

__device__ __forceinline__ void quantize_r0_block(const Theta& t, const uint32_t* __restrict__ slot,
                                                  uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, int64_t b) {
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
  __builtin_nontemporal_store(u32x2{packed[0], packed[1]}, cdst);   // written once, not read here again
  __builtin_nontemporal_store((uint8_t)S, sdst);
}

__global__ __launch_bounds__(256) void k_quantize_r0(Theta t, const uint32_t* __restrict__ slot, uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales, int64_t nblocks) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b < nblocks) quantize_r0_block(t, slot, codes, scales, b);
}

// ---------------------------------------------------------------------------------- rank > 0
// The rank terms go on the matrix cores. v_mfma_f32_32x32x1_2b_f32 adds the outer product of a
// 32-vector a and a 32-vector b into each of two independent 32 x 32 fp32 blocks, and rounds each
// element once, as an fma does: acc = fl32(acc + a*b). With one instruction per k, k ascending from
// an accumulator of +0, every element goes through exactly the scalar rounding sequence
// acc = fl32(acc + U[i,k] V[j,k]) (the bf16 x bf16 product is exact in fp32); s*W0 + acc is then
// one VALU fma. On gfx950 the instruction matched fmaf bit for bit on 8.2 M operand triples,
// subnormal results included. Since acc starts at +0 and every step rounds to nearest, neither acc
// nor w = fl32(s*W0 + acc) is ever -0.
//
// Operand and result placement of the instruction (lane L gives a to block L/32, row L%32 and b to
// block L/32, column L%32; result register v of lane l is block v/16, row 8*((v%16)/4) + 4*(l/32)
// + v%4, column l%32):
// * b = U[i0 + L%32][k] in both blocks, so result column l%32 is W row i0 + l%32;
// * a is V at a permuted column, chosen so that the 32 result registers of lane l are 32
//   consecutive columns of that W row: for block b and row m, the column is
//   c0 + 64*((m/4)%2) + 16*b + 4*(m/8) + m%4, where c0 is the wave's first column.
// Two instructions per k (the second 32 columns further on) give each lane 64 consecutive columns
// of one row -- four NVFP4 blocks, one 128-byte line of W0 -- with two independent accumulator
// chains; a wave's tile is 32 rows x 128 columns.
//
// Each wave (a workgroup of one wave) owns a 128-column strip and walks down its row tiles with a
// fixed stride, keeping the strip's V operands in registers for the whole walk. While the matrix
// cores and the VALU work on one tile, the U rows, row scales and W0 of the next tile are already
// on their way. The number of waves is what the chip holds at once, so there is no second round.
constexpr int kTileRows = 32;
constexpr int kWaveCols = 128;

// Passes of the rank > 0 kernels: the segment amax; the quantization (with ts in the slot); the
// rebuild written out as bf16; and the rebuild written out with its amax folded into the slot
// (the first pass of a staged quantization).
enum LowRankPass { kPassAmax = 0, kPassQuantize = 1, kPassReconstruct = 2, kPassAmaxStore = 3 };
constexpr bool takes_amax(int pass) { return pass == kPassAmax || pass == kPassAmaxStore; }
constexpr bool stores_weff(int pass) { return pass == kPassReconstruct || pass == kPassAmaxStore; }

typedef float f32x32 __attribute__((ext_vector_type(32)));

// Eight consecutive rank values k0 .. k0+7 of one U or V row as packed bf16 pairs (value k0 + 2i in
// the low half of word i); values at k >= r read as +0. VEC: r % 8 == 0 and the row 16-byte aligned.
template <bool VEC>
__device__ __forceinline__ u32x4 load_rank8(const uint16_t* __restrict__ row, int k0, int r) {
  if (VEC) return *reinterpret_cast<const u32x4*>(row + k0);
  uint32_t p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = (k0 + 2 * i < r) ? (uint32_t)row[k0 + 2 * i] : 0u;
    const uint32_t hi = (k0 + 2 * i + 1 < r) ? (uint32_t)row[k0 + 2 * i + 1] : 0u;
    p[i] = lo | (hi << 16);
  }
  return u32x4{p[0], p[1], p[2], p[3]};
}

// Eight rank steps k0 .. k0+7 (n of them valid, n >= 1) on both accumulator chains: b = U[row][k]
// and a = V[column][k] from packed bf16 pairs, k ascending.
__device__ __forceinline__ void rank8_steps(f32x32& acc0, f32x32& acc1, const u32x4& up, const u32x4& ap,
                                            const u32x4& bp, int n) {
  const uint32_t uw[4] = {up.x, up.y, up.z, up.w};
  const uint32_t aw[4] = {ap.x, ap.y, ap.z, ap.w};
  const uint32_t bw[4] = {bp.x, bp.y, bp.z, bp.w};
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    if (kk < n) {
      const float u = (kk & 1) ? bf16_hi(uw[kk >> 1]) : bf16_lo(uw[kk >> 1]);
      const float a = (kk & 1) ? bf16_hi(aw[kk >> 1]) : bf16_lo(aw[kk >> 1]);
      const float b = (kk & 1) ? bf16_hi(bw[kk >> 1]) : bf16_lo(bw[kk >> 1]);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x1f32(a, u, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x1f32(b, u, acc1, 0, 0, 0);
    }
  }
}

// What one tile needs from memory besides V: the first sixteen rank values of the lane's U row,
// its row scale and the 128 bytes of W0 behind its 64 columns.
struct TileIn {
  u32x4 u0, u1;
  uint32_t sbits;
  u32x4 w0[8];
};

// Issue a tile's loads. live == false (past the last tile): every load reads the first bytes of
// its matrix instead, so that a wave always has the same number of loads in flight and the
// waits for the current tile stay exact. Rows past N are clamped (their results are dropped);
// blocks past K read column 0.
template <bool VEC>
__device__ __forceinline__ TileIn tile_loads(const Theta& t, int row, int c0, bool live) {
  TileIn in;
  const int rowc = live ? min(row, t.N - 1) : 0;
  const uint16_t* ur = t.U + (size_t)rowc * t.r;
  const uint16_t* sp = t.s ? t.s + rowc : t.W0;
  in.sbits = *sp;
  in.u0 = load_rank8<VEC>(ur, 0, t.r);
  in.u1 = t.r > 8 ? load_rank8<VEC>(ur, 8, t.r) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int col = c0 + q * kBlock;
    const u32x4* src = reinterpret_cast<const u32x4*>(t.W0 + (size_t)rowc * t.K + (live && col < t.K ? col : 0));
    in.w0[2 * q] = src[0];
    in.w0[2 * q + 1] = src[1];
  }
  return in;
}

// The wave's largest |w| (fp32 bit patterns of |w| before the bf16 rounding; NaN patterns sort
// above every other) rounded once to bf16 and folded into the slot as the tensor scale
// fl32(amax / 2688) by atomicMax on its bits, as fold_tensor_scale does. bf16 rounding is
// monotone in |w|, so this is the largest rounded magnitude. The waves of a walk end almost
// together, and atomics on one address serialize, so a wave first reads the slot and skips the
// atomic when the slot already holds as much; a stale read only costs an atomic that changes
// nothing.
__device__ __forceinline__ void fold_wave_amax(uint32_t mx, uint32_t* slot, int lane) {
  mx = wave_max_u32(mx);
  const uint32_t m16 = mx ? f32_to_bf16_bits(__uint_as_float(mx)) << 16 : 0u;
  if (lane == 0 && m16) {
    const uint32_t tsb = __float_as_uint(tensor_scale_from_amax_bits(m16));
    if (__hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < tsb) atomicMax(slot, tsb);
  }
}

template <int PASS, bool VEC>
__device__ __forceinline__ void walk_tiles(const Theta& t, uint32_t* slot, uint8_t* __restrict__ codes,
                                           uint8_t* __restrict__ scales, uint16_t* __restrict__ out, int strips,
                                           int walkers) {
  const int lane = threadIdx.x;
  const int strip = blockIdx.x % strips;
  const int tiles_r = (t.N + kTileRows - 1) / kTileRows;
  const int j0 = strip * kWaveCols;
  const int c0 = j0 + 64 * (lane >> 5);           // the first of this lane's 64 result columns
  int rt = blockIdx.x / strips;                   // < tiles_r: walkers <= tiles_r

  uint32_t ts_bits = 0;
  if (PASS == kPassQuantize) {
    ts_bits = *slot;
    if (ts_bits >= 0x7F800000u) {                 // non-finite segment (ts NaN): NaN scales, zero codes
      for (; rt < tiles_r; rt += walkers) {
        const int row = rt * kTileRows + (lane & 31);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = c0 + q * kBlock;
          if (row < t.N && col < t.K) {
            *reinterpret_cast<u32x2*>(codes + (size_t)row * (t.K / 2) + col / 2) = u32x2{0u, 0u};
            scales[(size_t)row * (t.K / kBlock) + col / kBlock] = 0x7F;
          }
        }
      }
      return;
    }
  }

  // a operands: V rows at the permuted columns (clamped into the matrix; their results are
  // dropped), the first sixteen ranks held for the whole walk
  const int m = lane & 31, blk = lane >> 5;
  const int acol = j0 + 64 * ((m >> 2) & 1) + 16 * blk + 4 * (m >> 3) + (m & 3);
  const uint16_t* __restrict__ va = t.V + (size_t)min(acol, t.K - 1) * t.r;        // first instruction
  const uint16_t* __restrict__ vb = t.V + (size_t)min(acol + 32, t.K - 1) * t.r;   // second instruction
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  const u32x4 a0 = load_rank8<VEC>(va, 0, t.r), b0 = load_rank8<VEC>(vb, 0, t.r);
  const u32x4 a1 = t.r > 8 ? load_rank8<VEC>(va, 8, t.r) : zero4;
  const u32x4 b1 = t.r > 8 ? load_rank8<VEC>(vb, 8, t.r) : zero4;

  TileIn cur = tile_loads<VEC>(t, rt * kTileRows + (lane & 31), c0, true);
  uint32_t mx = 0;                                // amax pass: max |w| as fp32 bit patterns
  for (;;) {
    const int next = rt + walkers;
    const bool more = next < tiles_r;             // uniform
    const TileIn nxt = tile_loads<VEC>(t, next * kTileRows + (lane & 31), c0, more);
    const int row = rt * kTileRows + (lane & 31);
    const bool row_ok = row < t.N;

    f32x32 acc0, acc1;
#pragma unroll
    for (int v = 0; v < 32; ++v) {
      acc0[v] = 0.0f;
      acc1[v] = 0.0f;
    }
    rank8_steps(acc0, acc1, cur.u0, a0, b0, t.r);
    if (t.r > 8) rank8_steps(acc0, acc1, cur.u1, a1, b1, t.r - 8);
    for (int k0 = 16; k0 < t.r; k0 += 8) {        // ranks above 16, eight at a time
      const uint16_t* ur = t.U + (size_t)min(row, t.N - 1) * t.r;
      rank8_steps(acc0, acc1, load_rank8<VEC>(ur, k0, t.r), load_rank8<VEC>(va, k0, t.r),
                  load_rank8<VEC>(vb, k0, t.r), t.r - k0);
    }

    const float si = t.s ? bf16_bits_to_f32(cur.sbits) : 1.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int col = c0 + q * kBlock;
      const bool ok = row_ok && col < t.K;        // K % 16 == 0: a block is wholly inside or outside
      const uint32_t ww[8] = {cur.w0[2 * q].x, cur.w0[2 * q].y, cur.w0[2 * q].z, cur.w0[2 * q].w,
                              cur.w0[2 * q + 1].x, cur.w0[2 * q + 1].y, cur.w0[2 * q + 1].z, cur.w0[2 * q + 1].w};
      float w[kBlock];                            // fp32 s*W0 + acc, before the bf16 rounding
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const int e = (q & 1) * 16 + 2 * p;
        w[2 * p] = __builtin_fmaf(si, bf16_lo(ww[p]), q < 2 ? acc0[e] : acc1[e]);
        w[2 * p + 1] = __builtin_fmaf(si, bf16_hi(ww[p]), q < 2 ? acc0[e + 1] : acc1[e + 1]);
      }
      if (takes_amax(PASS)) {
        uint32_t bm = 0;
#pragma unroll
        for (int i = 0; i < kBlock; ++i) bm = max(bm, __float_as_uint(w[i]) & 0x7FFFFFFFu);
        mx = max(mx, ok ? bm : 0u);
      }
      if (PASS != kPassAmax) {
        uint32_t wp[kBlock / 2];
#pragma unroll
        for (int p = 0; p < 8; ++p) wp[p] = pack_bf16(w[2 * p], w[2 * p + 1]);
        if (PASS == kPassQuantize) {
          float wr[kBlock];                       // the bf16 values, all finite (else ts is NaN)
          float bamax = 0.0f;
#pragma unroll
          for (int p = 0; p < 8; ++p) {
            wr[2 * p] = bf16_lo(wp[p]);
            wr[2 * p + 1] = bf16_hi(wp[p]);
            bamax = __builtin_fmaxf(bamax, __builtin_fmaxf(__builtin_fabsf(wr[2 * p]), __builtin_fabsf(wr[2 * p + 1])));
          }
          if (ok) {
            uint32_t packed[2], S;
            quantize_values<false>(wr, bamax, ts_bits, packed, S);
            *reinterpret_cast<u32x2*>(codes + (size_t)row * (t.K / 2) + col / 2) = u32x2{packed[0], packed[1]};
            scales[(size_t)row * (t.K / kBlock) + col / kBlock] = (uint8_t)S;
          }
        } else if (ok) {
          u32x4* dst = reinterpret_cast<u32x4*>(out + (size_t)row * t.K + col);
          dst[0] = u32x4{wp[0], wp[1], wp[2], wp[3]};
          dst[1] = u32x4{wp[4], wp[5], wp[6], wp[7]};
        }
      }
    }
    if (!more) break;
    cur = nxt;
    rt = next;
  }
  if (takes_amax(PASS)) fold_wave_amax(mx, slot, lane);
}

template <int PASS, bool VEC>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void k_lowrank_walk(
    Theta t, uint32_t* slot, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, uint16_t* __restrict__ out,
    int strips, int walkers) {
  walk_tiles<PASS, VEC>(t, slot, codes, scales, out, strips, walkers);
}

// ------------------------------------------------------------------ rank 16: the pipelined walk
// The common case -- r = 16, U and V rows 16-byte aligned, N a multiple of 32 and K of 128, so
// that every tile is whole -- runs the same walk with the work of consecutive tiles overlapped.
// A lane's 64 columns are two halves with their own accumulator chains (A: the first 32, B: the
// last 32). In program order one step is
//   loads of tile t+1 | chain B(t) beside epilogue A(t) | chain A(t+1) beside epilogue B(t),
// so the matrix cores run one chain while the VALU finishes the other half, and the W0 of tile
// t+1 has a whole step to arrive. The loop body holds two steps with the two register sets
// swapped, so no loaded value is ever copied (a copy would wait for its load).
//
// The quantize pass rounds exactly as quantize_values<false> does. Its zero scale code uses
// (d, 1/d) = (1, 0) instead of a branch: q0 = w*0, r = fma(-q0, 1, w) = w, q = fma(w, 0, q0) is
// then a zero with the sign of w, which is what the exact rule gives. The quotient correction
// needs d and 1/d normal for every code, which holds for ts >= 2^-117; a segment with a smaller
// nonzero ts takes the per-block path of the walk above. An all-zero segment (ts = 0) divides
// its zero block maxima by 1 instead of 6 ts, which gives code 0 as well.
constexpr uint32_t kTsNormalFloor = 0x05000000u;   // 2^-117
// s_waitcnt operand: LDS/scalar counter 0, the vector-memory and export counters left at their
// maxima (no wait on them)
constexpr int kWaitLgkm0 = 0xC07F;

struct PipeIn {
  u32x4 u0, u1;        // U[row][0..15] of the lane's row
  uint32_t sbits;      // s[row]
  u32x4 w0[8];         // the tile's W0, coalesced: piece i of lane l is row 4i + l/16, bytes 16*(l%16)
};

// A tile's loads; live == false reads the first bytes of each matrix instead (see tile_loads). W0
// is read with whole rows per instruction (four rows of 256 bytes), not in the lanes' own
// layout: 64 lanes each touching a different line cost the vector L1 one lookup per lane, and
// at eight such loads per tile that lookup rate, not HBM, set the pace. The pieces go through
// LDS to their owners (stage_w0, own_w0).
__device__ __forceinline__ PipeIn pipe_loads(const Theta& t, int tile_row0, int j0, int lane, bool live) {
  PipeIn in;
  const int rowc = live ? tile_row0 + (lane & 31) : 0;
  const u32x4* ur = reinterpret_cast<const u32x4*>(t.U + (size_t)rowc * 16);
  in.u0 = ur[0];
  in.u1 = ur[1];
  in.sbits = *(t.s ? t.s + rowc : t.W0);
  const int r0 = live ? tile_row0 + (lane >> 4) : 0;
  const uint16_t* src = t.W0 + (size_t)r0 * t.K + (live ? j0 : 0) + 8 * (lane & 15);
#pragma unroll
  for (int i = 0; i < 8; ++i)                     // streamed: W0 is read once per pass
    in.w0[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (size_t)(live ? 4 * i : 0) * t.K));
  return in;
}

// The wave's LDS tile: 32 rows of 256 bytes, each padded by 16 bytes so that the owners' 16-byte
// reads (lane l: row l%32, bytes 128*(l/32) + 16j) and the staging writes are free of bank
// conflicts.
constexpr int kStageRowBytes = 2 * kWaveCols + 16;

__device__ __forceinline__ void stage_w0(uint8_t* lds, const PipeIn& in, int lane) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *reinterpret_cast<u32x4*>(lds + (4 * i + (lane >> 4)) * kStageRowBytes + 16 * (lane & 15)) = in.w0[i];
}

// The lane's 64 bytes of half `half` of the LDS tile (its columns 32*half .. 32*half+31).
__device__ __forceinline__ uint8_t* own_half(uint8_t* lds, int lane, int half) {
  return lds + (lane & 31) * kStageRowBytes + 128 * (lane >> 5) + 64 * half;
}

// The lane's four 16-byte W0 pieces of half `half`.
__device__ __forceinline__ void own_w0(uint8_t* lds, int lane, int half, u32x4 out[4]) {
  const uint8_t* row = own_half(lds, lane, half);
#pragma unroll
  for (int j = 0; j < 4; ++j) out[j] = *reinterpret_cast<const u32x4*>(row + 16 * j);
}

// The rebuilt tile, left in LDS by both halves, written out with whole rows per instruction (the
// transpose of stage_w0).
__device__ __forceinline__ void unstage_weff(const uint8_t* lds, uint16_t* out, int K, int tile_row0, int j0, int lane) {
  uint16_t* dst = out + (size_t)(tile_row0 + (lane >> 4)) * K + j0 + 8 * (lane & 15);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *reinterpret_cast<u32x4*>(dst + (size_t)(4 * i) * K) =
        *reinterpret_cast<const u32x4*>(lds + (4 * i + (lane >> 4)) * kStageRowBytes + 16 * (lane & 15));
}

// Non-negative finite fp32 -> E4M3FN code, as e4m3_encode_nonneg, without branches: both the
// normal rounding (keep 3 mantissa bits, round on the 20 dropped ones, ties to even, a carry may
// bump the exponent) and the uniform grid below 2^-6 (x * 512 rounded to an integer) are formed
// and one is selected; x >= 448 saturates. Equal to e4m3_encode_nonneg on every non-negative
// float up to +inf (checked exhaustively on the host).
__device__ __forceinline__ uint32_t e4m3_encode_select(float x) {
  const uint32_t b = __float_as_uint(x);
  const int e = (int)(b >> 23) - 127;
  const uint32_t mant = b & 0x7FFFFFu, keep = mant >> 20, rest = mant & 0xFFFFFu;
  const uint32_t up = (uint32_t)(rest > 0x80000u) | ((uint32_t)(rest == 0x80000u) & keep);
  const uint32_t normal = ((((uint32_t)(e + 7)) << 3) | keep) + up;
  const uint32_t sub = (uint32_t)__builtin_rintf(x * 512.0f);
  const uint32_t code = e < -6 ? sub : normal;
  return x >= 448.0f ? 0x7Eu : code;
}

__device__ __forceinline__ float bf16_of(const u32x4& p, int i) {      // element i (0..7) of 8 packed bf16
  const uint32_t w = (i >> 1) == 0 ? p.x : (i >> 1) == 1 ? p.y : (i >> 1) == 2 ? p.z : p.w;
  return (i & 1) ? bf16_hi(w) : bf16_lo(w);
}

// One phase of a step: the 16 rank steps of one chain (acc_chain, from +0, k ascending; b = u,
// a = V at the permuted columns) with the epilogue of one half (two blocks at columns col0 and
// col0 + 16 of `row`, from acc_epi and the half's W0 pieces own[0..3]) cut into 16 pieces, piece k
// issued right after rank step k. A scheduling fence after each piece keeps this order: each
// matrix instruction runs while the VALU works through the piece behind it. The amax pass
// rebuilds two elements per piece; the quantize pass rebuilds four elements per piece in pieces
// 0-7 (both blocks, keeping the bf16 values and the block maxima), sets each block's scale in
// pieces 8 and 9, and forms the quotients and codes of two or three element pairs per piece in
// pieces 10-15.
template <int PASS>
__device__ __forceinline__ void pipe_phase(f32x32& acc_chain, const u32x4& u0, const u32x4& u1, const u32x4& a0,
                                           const u32x4& a1, const f32x32& acc_epi, const u32x4 own[4], float si,
                                           size_t row, int col0, int K, float ts, float six_ts, uint32_t& mx,
                                           uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                           uint8_t* lds_half) {
  float wr[2 * kBlock];
  float bam[2] = {0.0f, 0.0f}, dd[2] = {1.0f, 1.0f}, yy[2] = {0.0f, 0.0f};
  uint32_t S[2] = {0u, 0u}, pk[4] = {0u, 0u, 0u, 0u};
  uint32_t wout[16];                              // the half's 32 bf16 values, when they are written out
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const u32x4& up = k < 8 ? u0 : u1;
    const u32x4& ap = k < 8 ? a0 : a1;
    const float u = bf16_of(up, k & 7), a = bf16_of(ap, k & 7);
    if (k == 0) {
#pragma unroll
      for (int v = 0; v < 32; ++v) acc_chain[v] = 0.0f;
    }
    acc_chain = __builtin_amdgcn_mfma_f32_32x32x1f32(a, u, acc_chain, 0, 0, 0);

    if (PASS != kPassQuantize) {                  // elements 2p, 2p+1 of block k/8, p = k%8
      const int blk = k >> 3, p = k & 7, e = 16 * blk + 2 * p;
      const float w0 = __builtin_fmaf(si, bf16_of(own[2 * blk + (p >> 2)], 2 * (p & 3)), acc_epi[e]);
      const float w1 = __builtin_fmaf(si, bf16_of(own[2 * blk + (p >> 2)], 2 * (p & 3) + 1), acc_epi[e + 1]);
      if (takes_amax(PASS)) mx = max(mx, max(__float_as_uint(w0) & 0x7FFFFFFFu, __float_as_uint(w1) & 0x7FFFFFFFu));
      if (stores_weff(PASS)) wout[k] = pack_bf16(w0, w1);
    } else if (k < 8) {                           // rebuild elements 2k, 2k+1 of both blocks
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const int e = 16 * blk + 2 * k;
        const float w0 = __builtin_fmaf(si, bf16_of(own[2 * blk + (k >> 2)], 2 * (k & 3)), acc_epi[e]);
        const float w1 = __builtin_fmaf(si, bf16_of(own[2 * blk + (k >> 2)], 2 * (k & 3) + 1), acc_epi[e + 1]);
        const uint32_t pr = pack_bf16(w0, w1);
        wr[e] = bf16_lo(pr);
        wr[e + 1] = bf16_hi(pr);
        bam[blk] = __builtin_fmaxf(bam[blk], __builtin_fmaxf(__builtin_fabsf(wr[e]), __builtin_fabsf(wr[e + 1])));
      }
    } else if (k < 10) {                          // the scale of block k-8
      const int blk = k - 8;
      S[blk] = e4m3_encode_select(bam[blk] / six_ts);
      const float d = e4m3_to_f32(S[blk]) * ts;
      dd[blk] = S[blk] ? d : 1.0f;
      yy[blk] = S[blk] ? 1.0f / d : 0.0f;
    } else {                                      // pairs P of piece k: 3,3,3,3,2,2 of the 16
      const int first = k < 14 ? 3 * (k - 10) : 12 + 2 * (k - 14);
      const int count = k < 14 ? 3 : 2;
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        if (i < count) {
          const int P = first + i, blk = P >> 3, wd = (P >> 2) & 1, j = P & 3, e = 16 * blk + 8 * wd + 2 * j;
          const float q0a = wr[e] * yy[blk], q0b = wr[e + 1] * yy[blk];
          const float qa = __builtin_fmaf(__builtin_fmaf(-q0a, dd[blk], wr[e]), yy[blk], q0a);
          const float qb = __builtin_fmaf(__builtin_fmaf(-q0b, dd[blk], wr[e + 1]), yy[blk], q0b);
          pk[2 * blk + wd] = cvt_fp4_pair(pk[2 * blk + wd], qa, qb, j);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if (PASS == kPassQuantize) {
    *reinterpret_cast<u32x4*>(codes + row * (size_t)(K / 2) + col0 / 2) = u32x4{pk[0], pk[1], pk[2], pk[3]};
    *reinterpret_cast<uint16_t*>(scales + row * (size_t)(K / kBlock) + col0 / kBlock) = (uint16_t)(S[0] | (S[1] << 8));
  }
  if (stores_weff(PASS)) {                        // back into the LDS tile, where this half's W0 was
    u32x4* dst = reinterpret_cast<u32x4*>(lds_half);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = u32x4{wout[4 * i], wout[4 * i + 1], wout[4 * i + 2], wout[4 * i + 3]};
  }
}

// acc = sum over k = 0 .. 15, ascending, of the outer products a_k (x) u_k (the first chain of a
// walk, with no epilogue beside it).
__device__ __forceinline__ void chain16(f32x32& acc, const u32x4& u0, const u32x4& u1, const u32x4& a0, const u32x4& a1) {
#pragma unroll
  for (int v = 0; v < 32; ++v) acc[v] = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k)
    acc = __builtin_amdgcn_mfma_f32_32x32x1f32(bf16_of(k < 8 ? a0 : a1, k & 7), bf16_of(k < 8 ? u0 : u1, k & 7), acc, 0,
                                               0, 0);
}

// One step of tile t. On entry X holds tile t's loads (arrived or in flight) and Y tile t+1's (in
// flight); acc0 holds chain A(t). The step waits for X's W0, stages it in LDS, keeps X's U row
// and row scale, and reissues X for tile t+2 (two tiles ahead), then runs chain B(t) beside
// epilogue A(t) and chain A(t+1) (from Y's U rows) beside epilogue B(t).
template <int PASS>
__device__ __forceinline__ void pipe_step(const Theta& t, PipeIn& X, const PipeIn& Y, f32x32& acc0, f32x32& acc1,
                                          const u32x4 (&va)[2], const u32x4 (&vb)[2], int tile_row0, int ahead_row0,
                                          bool ahead, int j0, int lane, uint8_t* lds, float ts, float six_ts,
                                          uint32_t& mx, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                          uint16_t* __restrict__ out) {
  stage_w0(lds, X, lane);
  const u32x4 u0 = X.u0, u1 = X.u1;
  const float si = t.s ? bf16_bits_to_f32(X.sbits) : 1.0f;
  X = pipe_loads(t, ahead_row0, j0, lane, ahead);
  const size_t row = (size_t)(tile_row0 + (lane & 31));
  const int c0 = j0 + 64 * (lane >> 5);
  // each half's W0 is read from LDS before its phase and waited for, so that no piece of the
  // phase waits on LDS
  u32x4 own[4];
  own_w0(lds, lane, 0, own);
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_sched_barrier(0);
  pipe_phase<PASS>(acc1, u0, u1, vb[0], vb[1], acc0, own, si, row, c0, t.K, ts, six_ts, mx, codes, scales,
                   own_half(lds, lane, 0));
  own_w0(lds, lane, 1, own);
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_sched_barrier(0);
  pipe_phase<PASS>(acc0, Y.u0, Y.u1, va[0], va[1], acc1, own, si, row, c0 + 32, t.K, ts, six_ts, mx, codes, scales,
                   own_half(lds, lane, 1));
  if (stores_weff(PASS)) unstage_weff(lds, out, t.K, tile_row0, j0, lane);
}

// One walk of a pipe wave over n row tiles of the 128-column strip at j0: tiles rt, rt + stride,
// ... The loads for tiles past the walk read the first bytes of each matrix instead (live ==
// false), so the number of loads in flight never depends on the walk's position.
template <int PASS>
__device__ __forceinline__ void pipe_walk(const Theta& t, uint32_t* slot, uint8_t* __restrict__ codes,
                                          uint8_t* __restrict__ scales, uint16_t* __restrict__ out, int j0, int rt,
                                          int stride, int n, float ts, float six_ts, int lane, uint8_t* lds) {
  const int m = lane & 31, blk = lane >> 5;
  const int acol = j0 + 64 * ((m >> 2) & 1) + 16 * blk + 4 * (m >> 3) + (m & 3);
  const u32x4* va_p = reinterpret_cast<const u32x4*>(t.V + (size_t)acol * 16);
  const u32x4* vb_p = reinterpret_cast<const u32x4*>(t.V + (size_t)(acol + 32) * 16);
  const u32x4 va[2] = {va_p[0], va_p[1]};
  const u32x4 vb[2] = {vb_p[0], vb_p[1]};

  uint32_t mx = 0;
  // tiles k = 0 .. n-1 of the walk; X and Y alternate between even and odd ones
  PipeIn X = pipe_loads(t, rt * kTileRows, j0, lane, true);
  PipeIn Y = pipe_loads(t, (rt + stride) * kTileRows, j0, lane, 1 < n);
  f32x32 acc0, acc1;
  chain16(acc0, X.u0, X.u1, va[0], va[1]);
  // A counted loop of two steps and one step after it. Written with an exit between the two steps,
  // the loop's control flow lets a Y step follow a Y step; the compiler's wait counts then take the
  // X set's loads as not in flight, or it swaps the sets by copying registers, and either way the
  // loads issued two tiles ahead are waited for one tile early.
  int k = 0;
  for (; k + 1 < n; k += 2) {
    pipe_step<PASS>(t, X, Y, acc0, acc1, va, vb, rt * kTileRows, (rt + 2 * stride) * kTileRows, k + 2 < n, j0, lane,
                    lds, ts, six_ts, mx, codes, scales, out);
    rt += stride;
    pipe_step<PASS>(t, Y, X, acc0, acc1, va, vb, rt * kTileRows, (rt + 2 * stride) * kTileRows, k + 3 < n, j0, lane,
                    lds, ts, six_ts, mx, codes, scales, out);
    rt += stride;
  }
  if (k < n)
    pipe_step<PASS>(t, X, Y, acc0, acc1, va, vb, rt * kTileRows, (rt + 2 * stride) * kTileRows, false, j0, lane, lds,
                    ts, six_ts, mx, codes, scales, out);
  if (takes_amax(PASS)) fold_wave_amax(mx, slot, lane);
}

template <int PASS>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void k_lowrank_pipe(
    Theta t, uint32_t* slot, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, uint16_t* __restrict__ out,
    int strips, int walkers) {
  const int lane = threadIdx.x;
  const int strip = blockIdx.x % strips;
  const int tiles_r = t.N / kTileRows;
  const int rt = blockIdx.x / strips;             // < tiles_r: walkers <= tiles_r

  float ts = 0.0f, six_ts = 1.0f;
  if (PASS == kPassQuantize) {
    const uint32_t ts_bits = *slot;
    if (ts_bits >= 0x7F800000u || (ts_bits != 0u && ts_bits < kTsNormalFloor)) {
      // a non-finite segment, or one too small for the correction: the walk's per-block path
      walk_tiles<kPassQuantize, true>(t, slot, codes, scales, nullptr, strips, walkers);
      return;
    }
    ts = __uint_as_float(ts_bits);
    six_ts = ts_bits ? 6.0f * ts : 1.0f;
  }
  __shared__ __align__(16) uint8_t lds[kTileRows * kStageRowBytes];
  pipe_walk<PASS>(t, slot, codes, scales, out, strip * kWaveCols, rt, walkers, (tiles_r - rt + walkers - 1) / walkers,
                  ts, six_ts, lane, lds);
}

// ------------------------------------------------------------------------- batches of bundles
// The staged quantization of up to kMaxBatch theta bundles in three launches (the slot resets, the
// rebuild of every whole-tile rank-16 bundle, the quantization of every bundle) instead of three
// per bundle: a model's loader calls it once per layer. A bundle's result is the single staged
// call's bit for bit: each element goes through the same arithmetic, and the amax fold is a max.
constexpr int kMaxBatch = ATTNQ_MAX_BATCH;

// An element of a per-bundle array picked by a wave-uniform index, without dynamic indexing (which
// would copy the kernel argument to scratch memory).
template <typename T>
__device__ __forceinline__ T pick(const T (&a)[kMaxBatch], int i) {
  T v = a[0];
#pragma unroll
  for (int k = 1; k < kMaxBatch; ++k) v = (k == i) ? a[k] : v;
  return v;
}

__device__ __forceinline__ Theta pick_theta(const Theta (&a)[kMaxBatch], int i) {
  Theta v = a[0];
#pragma unroll
  for (int k = 1; k < kMaxBatch; ++k)
    if (k == i) v = a[k];
  return v;
}

struct SlotList {
  uint32_t* slot[kMaxBatch];
  int n;
};

__global__ void k_zero_slots(SlotList l) {
  if (blockIdx.x == 0 && (int)threadIdx.x < l.n) *pick(l.slot, threadIdx.x) = 0u;
}

// Rebuild pass of the batch: the bundles' grids of the single call (strips x walkers one-wave
// workgroups each, as many as the device holds at once) laid end to end in one launch. The device
// runs them in that order, so a bundle's walks start as the previous bundle's finish, without the
// gap and the ramp of a launch, and each bundle keeps the single call's access pattern (the walkers
// of all strips on the same row tile at about the same time, so whole rows are read together).
struct PipeBatch {
  Theta t[kMaxBatch];
  uint32_t* slot[kMaxBatch];
  uint16_t* out[kMaxBatch];
  int wg_end[kMaxBatch];        // workgroups of bundles 0 .. i
  int strips[kMaxBatch], walkers[kMaxBatch];
  int n;
};

template <int PASS>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void k_lowrank_pipe_batch(PipeBatch b) {
  static_assert(PASS == kPassAmax || PASS == kPassAmaxStore || PASS == kPassReconstruct, "no quantize pass in a batch");
  __shared__ __align__(16) uint8_t lds[kTileRows * kStageRowBytes];
  const int lane = threadIdx.x;
  const int wg = blockIdx.x;
  int i = 0;
#pragma unroll
  for (int k = 0; k < kMaxBatch - 1; ++k) i += (k < b.n - 1 && wg >= b.wg_end[k]) ? 1 : 0;
  const int local = wg - (i ? pick(b.wg_end, i - 1) : 0);
  const Theta t = pick_theta(b.t, i);
  const int strips = pick(b.strips, i), walkers = pick(b.walkers, i);
  const int strip = local % strips, rt = local / strips;
  const int tiles_r = t.N / kTileRows;
  pipe_walk<PASS>(t, pick(b.slot, i), nullptr, nullptr, pick(b.out, i), strip * kWaveCols, rt, walkers,
                  (tiles_r - rt + walkers - 1) / walkers, 0.0f, 1.0f, lane, lds);
}

// Quantize pass of the batch: every bundle's 16-element blocks in one grid (bundle by bundle, each
// bundle starting on a workgroup of its own, so that the bundle index is uniform and its picks are
// scalar), from W_eff in the workspace (rank > 0) or from s and W0 (rank 0), with the bundle's slot
// as ts.
struct QuantBatch {
  Theta t[kMaxBatch];           // rank 0 form: W_eff, or W0 and s
  const uint32_t* slot[kMaxBatch];
  uint8_t* codes[kMaxBatch];
  uint8_t* scales[kMaxBatch];
  int64_t nblocks[kMaxBatch];
  int wg_end[kMaxBatch];        // workgroups of bundles 0 .. i
  int n;
};

__global__ __launch_bounds__(256) void k_quantize_r0_batch(QuantBatch q) {
  const int wg = blockIdx.x;
  int i = 0;
#pragma unroll
  for (int k = 0; k < kMaxBatch - 1; ++k) i += (k < q.n - 1 && wg >= q.wg_end[k]) ? 1 : 0;
  const int64_t b = (int64_t)(wg - (i ? pick(q.wg_end, i - 1) : 0)) * 256 + threadIdx.x;
  if (b < pick(q.nblocks, i))
    quantize_r0_block(pick_theta(q.t, i), pick(q.slot, i), pick(q.codes, i), pick(q.scales, i), b);
}

Theta to_theta(const attnq_theta& t) { return Theta{t.W0, t.s, t.U, t.V, t.N, t.K, t.r}; }

// Waves of a walking kernel resident on the device at once (occupancy x compute units), per device
// and kernel (slot).
template <typename Kernel>
int walk_capacity(Kernel kernel, std::atomic<int>* cache) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1024;
  int c = cache[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 64, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || per_cu < 1 || cus < 1)
      return 1024;
    c = per_cu * cus;
    cache[dev].store(c, std::memory_order_relaxed);
  }
  return c;
}

template <int PASS, bool VEC>
void launch_walk(const Theta& t, uint32_t* slot, uint8_t* codes, uint8_t* scales, uint16_t* out, hipStream_t stream) {
  static std::atomic<int> cap[64];
  const int tiles_r = (t.N + kTileRows - 1) / kTileRows;
  const int strips = (t.K + kWaveCols - 1) / kWaveCols;
  const int walkers = max(1, min(tiles_r, walk_capacity(k_lowrank_walk<PASS, VEC>, cap) / strips));
  k_lowrank_walk<PASS, VEC><<<(unsigned)(strips * walkers), 64, 0, stream>>>(t, slot, codes, scales, out, strips, walkers);
}

template <int PASS>
void launch_pipe(const Theta& t, uint32_t* slot, uint8_t* codes, uint8_t* scales, uint16_t* out, hipStream_t stream) {
  static std::atomic<int> cap[64];
  const int tiles_r = t.N / kTileRows;
  const int strips = t.K / kWaveCols;
  const int walkers = max(1, min(tiles_r, walk_capacity(k_lowrank_pipe<PASS>, cap) / strips));
  k_lowrank_pipe<PASS><<<(unsigned)(strips * walkers), 64, 0, stream>>>(t, slot, codes, scales, out, strips, walkers);
}

template <int PASS>
void launch_lowrank(const Theta& t, uint32_t* slot, uint8_t* codes, uint8_t* scales, uint16_t* out, hipStream_t stream) {
  const bool vec = t.r % 8 == 0 && reinterpret_cast<uintptr_t>(t.U) % 16 == 0 && reinterpret_cast<uintptr_t>(t.V) % 16 == 0;
  if (t.r == 16 && vec && t.N % kTileRows == 0 && t.K % kWaveCols == 0)
    launch_pipe<PASS>(t, slot, codes, scales, out, stream);
  else if (vec)
    launch_walk<PASS, true>(t, slot, codes, scales, out, stream);
  else
    launch_walk<PASS, false>(t, slot, codes, scales, out, stream);
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

int64_t quantize_staged_workspace_bytes(int32_t N, int32_t K, int32_t r) {
  return (r > 0 && N > 0 && K > 0) ? (int64_t)N * K * 2 : 0;
}

hipError_t launch_quantize_staged(const attnq_theta& th, uint8_t* codes, uint8_t* scales, float* tensor_scale,
                                  void* workspace, hipStream_t stream) {
  const Theta t = to_theta(th);
  const int64_t nblocks = (int64_t)th.N * (th.K / kBlock);
  if (t.r == 0 || nblocks == 0) return launch_quantize(th, codes, scales, tensor_scale, stream);
  uint32_t* slot = reinterpret_cast<uint32_t*>(tensor_scale);
  uint16_t* weff = static_cast<uint16_t*>(workspace);
  k_zero_slot<<<1, 64, 0, stream>>>(slot);
  launch_lowrank<kPassAmaxStore>(t, slot, nullptr, nullptr, weff, stream);
  const Theta staged{weff, nullptr, nullptr, nullptr, t.N, t.K, 0};   // W_eff, passed through
  k_quantize_r0<<<(unsigned)((nblocks + 255) / 256), 256, 0, stream>>>(staged, slot, codes, scales, nblocks);
  return hipGetLastError();
}

int64_t quantize_staged_batch_workspace_bytes(const attnq_theta* th, int count) {
  int64_t total = 0;
  for (int i = 0; i < count; ++i) total += (quantize_staged_workspace_bytes(th[i].N, th[i].K, th[i].r) + 255) / 256 * 256;
  return total;
}

hipError_t launch_quantize_staged_batch(const attnq_theta* th, uint8_t* const* codes, uint8_t* const* scales,
                                        float* const* tensor_scale, int count, void* workspace, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  SlotList slots{};
  slots.n = count;
  PipeBatch pb{};
  QuantBatch qb{};
  uint16_t* weff[kMaxBatch] = {};
  int64_t off = 0;
  int wgs = 0, qwgs = 0;
  for (int i = 0; i < count; ++i) {
    const Theta t = to_theta(th[i]);
    uint32_t* slot = reinterpret_cast<uint32_t*>(tensor_scale[i]);
    slots.slot[i] = slot;
    const int64_t need = quantize_staged_workspace_bytes(t.N, t.K, t.r);
    weff[i] = need > 0 ? reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(workspace) + off) : nullptr;
    off += (need + 255) / 256 * 256;
    const int64_t nblocks = (int64_t)t.N * (t.K / kBlock);
    if (nblocks > 0) {
      qwgs += (int)((nblocks + 255) / 256);
      qb.t[qb.n] = t.r > 0 ? Theta{weff[i], nullptr, nullptr, nullptr, t.N, t.K, 0} : Theta{t.W0, t.s, nullptr, nullptr, t.N, t.K, 0};
      qb.slot[qb.n] = slot;
      qb.codes[qb.n] = codes[i];
      qb.scales[qb.n] = scales[i];
      qb.nblocks[qb.n] = nblocks;
      qb.wg_end[qb.n] = qwgs;
      ++qb.n;
    }
    const bool vec = t.r % 8 == 0 && reinterpret_cast<uintptr_t>(t.U) % 16 == 0 && reinterpret_cast<uintptr_t>(t.V) % 16 == 0;
    if (nblocks > 0 && t.r == 16 && vec && t.N % kTileRows == 0 && t.K % kWaveCols == 0) {
      static std::atomic<int> cap[64];
      const int strips = t.K / kWaveCols;
      const int walkers = max(1, min(t.N / kTileRows, walk_capacity(k_lowrank_pipe_batch<kPassAmaxStore>, cap) / strips));
      wgs += strips * walkers;
      pb.t[pb.n] = t;
      pb.slot[pb.n] = slot;
      pb.out[pb.n] = weff[i];
      pb.wg_end[pb.n] = wgs;
      pb.strips[pb.n] = strips;
      pb.walkers[pb.n] = walkers;
      ++pb.n;
    }
  }
  k_zero_slots<<<1, 64, 0, stream>>>(slots);
  if (pb.n > 0) k_lowrank_pipe_batch<kPassAmaxStore><<<(unsigned)wgs, 64, 0, stream>>>(pb);
  for (int i = 0; i < count; ++i) {                 // bundles outside the rank-16 batch, one by one
    const Theta t = to_theta(th[i]);
    const int64_t nblocks = (int64_t)t.N * (t.K / kBlock);
    bool in_pb = false;
    for (int k = 0; k < pb.n; ++k) in_pb |= pb.out[k] == weff[i] && weff[i] != nullptr;
    if (nblocks == 0 || in_pb) continue;
    uint32_t* slot = reinterpret_cast<uint32_t*>(tensor_scale[i]);
    if (t.r > 0) {
      launch_lowrank<kPassAmaxStore>(t, slot, nullptr, nullptr, weff[i], stream);
    } else {
      const int64_t want = (nblocks + 255) / 256;
      k_amax_r0<<<(unsigned)(want < 4096 ? want : 4096), 256, 0, stream>>>(t, slot, nblocks);
    }
  }
  if (qb.n > 0) k_quantize_r0_batch<<<(unsigned)qwgs, 256, 0, stream>>>(qb);
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
