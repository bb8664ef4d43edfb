// Small-M NVFP4 product Y = X * W^T for M <= 16 token rows: speculative verification of
// gamma = 3 drafted tokens plus one ("Throughput", "Speculative decoding") and batch 8.
//
// M <= 4 with rows of at most 192 chunks (6144 elements) goes to the batch-1 walk first
// (k_gemm_nvfp4_tokens, next to the GEMV kernels), which measured faster there; the matrix-core
// kernels below take longer rows and M > 4.
//
// Matrix-core path, v_mfma_f32_16x16x32_bf16. Operand layout for lane l = 16 g + i (checked on
// gfx950): A[i][8 g + e], B[8 g + e][i] for e = 0..7, and D[4 g + v][i] for v = 0..3.
//
// Weights (B operand). Lane (g, i) of row tile t owns code bytes 16 g .. 16 g + 15 and 64 + 16 g ..
// 64 + 16 g + 15 of weight row 16 t + i in every 256-element superchunk (128 code bytes), so each
// 16-byte load instruction reads one contiguous 64-byte half line per row. The K order inside an
// MFMA is free as long as A and B agree: dword m of the lane's 32 bytes feeds MFMA m (m = 0..7)
// and covers superchunk positions 32 g + 8 (m % 4) + 128 (m / 4) + e, in block
// 2 g + (m / 2) % 2 + 8 (m / 4).
//
// M <= 4, block scales as MFMA rows (k_gemm_small_m_mfma). Codes are decoded to bf16 without
// their scale (v_cvt_scalef32_pk_bf16_fp4, exact). An MFMA sums over all 32 of its K positions,
// which belong to four different scale blocks (one per lane group g); to keep the blocks apart,
// the A row index carries (token, block slot): A[4 tau + b][8 g + e] = X[token tau][pos] when
// b == g and 0 otherwise. After MFMAs 2 h and 2 h + 1, output row 4 tau + v holds the
// exact-product fp32 partial dot product of token tau over the block lane group v holds in pair h,
// 2 v + h % 2 + 8 (h / 2), and lane (tau, row) applies that block's E4M3 scale with one FMA per v. (The template also runs
// P = ceil(M / 4) passes over the same decoded weights for larger M; the launcher uses P = 1.)
//
// 4 < M <= 16, tokens as MFMA rows (k_gemm_small_m_scaled). Codes are decoded to fp32,
// multiplied by their E4M3 scale and packed to bf16, which is exact: a code value times an E4M3
// value has at most 6 significant bits and lies in [2^-10, 2688]. All MFMAs of a row tile then
// accumulate into one 16 x 16 tile of (token, row) dot products.
//
// In both, every product is exact and only the fp32 summation order differs from a plain dot
// product; the tensor scale is applied last. A workgroup owns 2 x 16 weight rows; its waves split
// the superchunks of K, keep the next superchunk's weights in flight while computing the current
// one, and meet in LDS at the end. Rows past N and tokens past M are clamped or masked and never
// stored. The M <= 4 kernel also loads each superchunk's X together with its weights, one
// superchunk ahead: load counters complete in order, so X loaded inside the compute step (after
// the next superchunk's weight loads) would make every wait for X a wait for those weights too.
#include <atomic>

#include "attnq_device.h"
#include "launch.h"

namespace attnq {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kSuper = 256;        // K elements per superchunk: 128 code bytes and 16 scale bytes per row
constexpr int kMaxWaves = 12;      // K split: waves of one workgroup over the same rows (the launch bound
                                   // of 768 threads leaves 168 VGPRs per lane for the operand buffers)

// 8 E2M1 codes (even element in the low nibble) -> 8 bf16, exact.
__device__ __forceinline__ bf16x8 decode8(uint32_t w) {
  const u32x4 p = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3))};
  return __builtin_bit_cast(bf16x8, p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint32_t word(const u32x4& v, int j) {
  return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

// E4M3 byte h of a dword -> fp32 (h is a constant after unrolling).
__device__ __forceinline__ float e4m3_byte(uint32_t w, int h) {
  switch (h) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8((int)w, 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8((int)w, 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8((int)w, 2);
    default: return __builtin_amdgcn_cvt_f32_fp8((int)w, 3);
  }
}

// The 16 scale bytes of one row and superchunk. Rows start 16-byte aligned only when K % 256 == 0;
// otherwise (K % 32 == 0 keeps them 2-byte aligned) the bytes are gathered as halfwords.
__device__ __forceinline__ u32x4 load_scales16(const uint8_t* p, bool aligned16) {
  if (aligned16) return *reinterpret_cast<const u32x4*>(p);
  const uint16_t* q = reinterpret_cast<const uint16_t*>(p);
  return u32x4{q[0] | ((uint32_t)q[1] << 16), q[2] | ((uint32_t)q[3] << 16), q[4] | ((uint32_t)q[5] << 16),
               q[6] | ((uint32_t)q[7] << 16)};
}

template <int RT, int P>
__global__ __launch_bounds__(64 * kMaxWaves) void k_gemm_small_m_mfma(const uint8_t* __restrict__ codes,
                                                                     const uint8_t* __restrict__ scales,
                                                                     const float* __restrict__ tensor_scale,
                                                                     SegTable segs, const uint16_t* __restrict__ X,
                                                                     int M, int ldx, float* __restrict__ Y, int ldy,
                                                                     int N, int K, int per) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, ks = blockDim.x >> 6;
  const int g = lane >> 4, i = lane & 15;
  const int row0 = blockIdx.x * (16 * RT);
  const size_t code_pitch = (size_t)K >> 1, scale_pitch = (size_t)K >> 4;
  const bool scales_a16 = (scale_pitch & 15) == 0;

  const uint8_t* crow[RT];     // this lane's 32-byte slice of superchunk 0 of its row
  const uint8_t* srow[RT];     // the row's scales
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int row = min(row0 + 16 * t + i, N - 1);
    crow[t] = codes + (size_t)row * code_pitch + 16 * g;
    srow[t] = scales + (size_t)row * scale_pitch;
  }
  // A operand source: lane (g, i) carries token 4 p + (i >> 2) when (i & 3) == g. X is read through
  // a buffer resource bounded to its extent: the other lanes use an offset past the end, which
  // returns zeros without a memory request, so every X load is unconditional.
  bool act[P];
  const uint16_t* xrow[P];
  const int x_bytes = ((M - 1) * ldx + K) * 2;
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(X), (short)0, x_bytes,
                                                                        0x00020000);
  int xoff[P];                 // byte offset of this lane's X piece in superchunk 0
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int tok = 4 * p + (i >> 2);
    act[p] = ((i & 3) == g) && tok < M;
    xrow[p] = X + (size_t)min(tok, M - 1) * ldx;
    xoff[p] = act[p] ? (tok * ldx + 32 * g) * 2 : x_bytes;
  }

  float acc[P][RT];
#pragma unroll
  for (int p = 0; p < P; ++p)
#pragma unroll
    for (int t = 0; t < RT; ++t) acc[p][t] = 0.0f;

  const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
  const int nsc = K / kSuper;
  const int s_begin = wave * per, s_end = min(nsc, s_begin + per);

  // Code and scale loads of superchunk sc into one of two register buffers, then its X pieces
  // (MFMAs 2 h and 2 h + 1 take positions 32 g + 16 (h % 2) + 128 (h / 2) .. + 15). Each
  // superchunk's X is issued with its weights, ahead of the next superchunk's loads, so that the
  // wait for it (counters complete in order) never waits for the next superchunk's weights.
  auto load_w = [&](u32x4 (&cw)[RT][2], u32x4 (&sw)[RT], u32x4 (&xa)[P][4][2], int sc) {
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const u32x4* cp = reinterpret_cast<const u32x4*>(crow[t] + (size_t)sc * (kSuper / 2));
      cw[t][0] = __builtin_nontemporal_load(cp);
      cw[t][1] = __builtin_nontemporal_load(cp + 4);
      sw[t] = load_scales16(srow[t] + (size_t)sc * (kSuper / kBlock), scales_a16);
    }
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int o = xoff[p] + (sc * kSuper + 16 * (h & 1) + 128 * (h >> 1)) * 2;
        xa[p][h][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xres, o, 0, 0));
        xa[p][h][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xres, o + 16, 0, 0));
      }
  };
  auto compute = [&](const u32x4 (&cw)[RT][2], const u32x4 (&sw)[RT], const u32x4 (&xa)[P][4][2], int sc) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const bf16x8 b0 = decode8(word(cw[t][h >> 1], 2 * (h & 1)));
        const bf16x8 b1 = decode8(word(cw[t][h >> 1], 2 * (h & 1) + 1));
        // scale of the block that lane group v holds in pair h: 2 v + (h & 1) + 8 (h >> 1)
        float s[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int b = 2 * v + (h & 1) + 8 * (h >> 1);
          s[v] = e4m3_byte(word(sw[t], b >> 2), b & 3);
        }
#pragma unroll
        for (int p = 0; p < P; ++p) {
          f32x4 d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[p][h][0]), b0, zero4, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[p][h][1]), b1, d, 0, 0, 0);
          float a = acc[p][t];
          a = __builtin_fmaf(d.x, s[0], a);
          a = __builtin_fmaf(d.y, s[1], a);
          a = __builtin_fmaf(d.z, s[2], a);
          a = __builtin_fmaf(d.w, s[3], a);
          acc[p][t] = a;
        }
      }
    }
  };
  // Two-stage pipeline: the weights and X of the next superchunk are in flight while this one computes.
  if (s_begin < s_end) {
    u32x4 cwa[RT][2], swa[RT], cwb[RT][2], swb[RT];
    u32x4 xaa[P][4][2], xab[P][4][2];
    load_w(cwa, swa, xaa, s_begin);
    for (int sc = s_begin; sc < s_end; sc += 2) {
      if (sc + 1 < s_end) load_w(cwb, swb, xab, sc + 1);
      compute(cwa, swa, xaa, sc);
      if (sc + 1 < s_end) {
        if (sc + 2 < s_end) load_w(cwa, swa, xaa, sc + 2);
        compute(cwb, swb, xab, sc + 1);
      }
    }
  }

  // Tail: 32-element chunks past the last full superchunk (K % 256 in {32, ..., 224}). Lane
  // group g takes dword g of the chunk's 16 code bytes (positions 8 g .. 8 g + 7, block g / 2);
  // output row 4 tau + v then holds block v / 2 of the chunk.
  const int nch = K >> 5;
  for (int ch = nsc * (kSuper / kChunkElems) + wave; ch < nch; ch += ks) {
    u32x4 xt[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      xt[p] = u32x4{0u, 0u, 0u, 0u};
      if (act[p]) xt[p] = *reinterpret_cast<const u32x4*>(xrow[p] + (size_t)ch * kChunkElems + 8 * g);
    }
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const uint8_t* cbase = crow[t] - 16 * g;
      const uint32_t w = *reinterpret_cast<const uint32_t*>(cbase + (size_t)ch * 16 + 4 * g);
      const uint32_t sv = *reinterpret_cast<const uint16_t*>(srow[t] + (size_t)ch * 2);
      const float s_lo = __builtin_amdgcn_cvt_f32_fp8((int)sv, 0), s_hi = __builtin_amdgcn_cvt_f32_fp8((int)sv, 1);
      const bf16x8 b = decode8(w);
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const f32x4 d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xt[p]), b, zero4, 0, 0, 0);
        float a = acc[p][t];
        a = __builtin_fmaf(d.x, s_lo, a);
        a = __builtin_fmaf(d.y, s_lo, a);
        a = __builtin_fmaf(d.z, s_hi, a);
        a = __builtin_fmaf(d.w, s_hi, a);
        acc[p][t] = a;
      }
    }
  }

  __shared__ float part[kMaxWaves - 1][P][RT][64];
  if (ks > 1) {
    if (wave > 0) {
#pragma unroll
      for (int p = 0; p < P; ++p)
#pragma unroll
        for (int t = 0; t < RT; ++t) part[wave - 1][p][t][lane] = acc[p][t];
    }
    __syncthreads();
    if (wave != 0) return;
    for (int w = 0; w < ks - 1; ++w)
#pragma unroll
      for (int p = 0; p < P; ++p)
#pragma unroll
        for (int t = 0; t < RT; ++t) acc[p][t] += part[w][p][t][lane];
  }
  // lane (g, i): token 4 p + g, weight row row0 + 16 t + i
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int row = row0 + 16 * t + i;
    if (row < N) {
      const float ts = tensor_scale[segment_of(segs, row)];
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int m = 4 * p + g;
        if (m < M) Y[(size_t)m * ldy + row] = acc[p][t] * ts;
      }
    }
  }
}

// 8 E2M1 codes times their E4M3 block scale s -> 8 bf16. Exact: a code value times an E4M3
// value has at most 6 significant bits and lies in [2^-10, 2688].
__device__ __forceinline__ bf16x8 decode8_scaled(uint32_t w, float s) {
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const auto f = j == 0 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0)
                 : j == 1 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1)
                 : j == 2 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2)
                          : __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    const bf16x2v p = {(__bf16)(f[0] * s), (__bf16)(f[1] * s)};
    const uint32_t u = __builtin_bit_cast(uint32_t, p);
    if (j == 0) r.x = u; else if (j == 1) r.y = u; else if (j == 2) r.z = u; else r.w = u;
  }
  return __builtin_bit_cast(bf16x8, r);
}

// fp16 operands for the staged-X kernels (slices and walking strips). Decoding to bf16 costs two
// VALU instructions per weight (a convert to fp32 pairs, a multiply per value and a pack); in fp16
// it is one convert per pair at scale 1 and one packed multiply by the block scale, which is exact
// for the same reason (the product's 6 significant bits and its range [2^-10, 2688] fit fp16's
// normal range). X then has to be fp16 too, and a bf16 value is exactly an fp16 one once scaled by
// a power of two into fp16's normal range: this holds for a token's values in one staged window when
// all are finite and every nonzero one lies within 2^29 of the window's largest. The workgroup
// checks that while staging; if it holds for every token it stores each token's window scaled by
// 2^(15 - e_max) as fp16, and multiplies that token's sums by the inverse power of two, which is
// exact: every product and partial sum is the bf16 computation's times a power of two, and the
// exponent limits below keep every value normal in fp32. Otherwise the window stays bf16.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kF16Span = 29;             // octaves between a window's largest value and its smallest nonzero
constexpr int kF16MinExp = 127 - 75;     // the largest value's biased exponent: 2^-75 .. 2^105
constexpr int kF16MaxExp = 127 + 105;

__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }

// 8 E2M1 codes times their E4M3 block scale (both fp16 halves of s2) -> 8 fp16, exact.
__device__ __forceinline__ f16x8 decode8_f16(uint32_t w, f16x2 s2) {
  const u32x4 r = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2)};
  return __builtin_bit_cast(f16x8, r);
}

// E4M3 byte h of a dword, in both halves of an fp16 pair (exact: E4M3 values are fp16 normals).
__device__ __forceinline__ f16x2 e4m3_pair(uint32_t w, int h) {
  const _Float16 v = (_Float16)(h == 0 ? __builtin_amdgcn_cvt_f32_fp8((int)w, 0) : __builtin_amdgcn_cvt_f32_fp8((int)w, 1));
  return f16x2{v, v};
}

// Largest biased exponent of 8 bf16 values; bad is set for inf, NaN and bf16 subnormals.
__device__ __forceinline__ int piece_emax(const u32x4& v, int& bad) {
  int e = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t h = (word(v, j >> 1) >> (16 * (j & 1))) & 0x7FFFu;
    const int f = (int)(h >> 7);
    e = max(e, f);
    bad |= (f == 255) | ((f == 0) & (h != 0));
  }
  return e;
}

// Whether every nonzero value of the piece lies within kF16Span octaves of the token's largest.
__device__ __forceinline__ int piece_out_of_span(const u32x4& v, int emax) {
  int bad = emax != 0 && (emax < kF16MinExp || emax > kF16MaxExp);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t h = (word(v, j >> 1) >> (16 * (j & 1))) & 0x7FFFu;
    bad |= (h != 0) & ((int)(h >> 7) < emax - kF16Span);
  }
  return bad;
}

__device__ __forceinline__ float pow2_biased(int e) { return __builtin_bit_cast(float, (uint32_t)e << 23); }

// 8 bf16 values times 2^(15 - (emax - 127)) -> 8 fp16 (exact under piece_out_of_span's conditions).
__device__ __forceinline__ u32x4 piece_to_f16(const u32x4& v, int emax) {
  const float sc = emax == 0 ? 1.0f : pow2_biased(127 + 142 - emax);
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w = word(v, j);
    const auto h = __builtin_amdgcn_cvt_pkrtz(__builtin_bit_cast(float, w << 16) * sc,
                                              __builtin_bit_cast(float, w & 0xFFFF0000u) * sc);
    const uint32_t u = __builtin_bit_cast(uint32_t, h);
    if (j == 0) r.x = u; else if (j == 1) r.y = u; else if (j == 2) r.z = u; else r.w = u;
  }
  return r;
}

// The inverse of piece_to_f16's factor, applied to a token's sums.
__device__ __forceinline__ float f16_unscale(int emax) { return emax == 0 ? 1.0f : pow2_biased(emax - 15); }

// A workgroup's X pieces before they go to LDS: tok[j] is piece j's token, or -1 for a piece that
// is stored as zero. e[16] (LDS) receives each token's largest biased exponent. Returns, the same
// for every thread, whether the window takes the fp16 operands; the pieces are then converted.
template <int NP>
__device__ __forceinline__ bool stage_f16(u32x4 (&xv)[NP], const int (&tok)[NP], int* e) {
  if (threadIdx.x < 16) e[threadIdx.x] = 0;
  __syncthreads();
  int bad = 0;
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    if (tok[j] >= 0) {
      const int em = piece_emax(xv[j], bad);
      if (em != 0) atomicMax(&e[tok[j]], em);
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NP; ++j)
    if (tok[j] >= 0) bad |= piece_out_of_span(xv[j], e[tok[j]]);
  const bool f16 = __syncthreads_or(bad) == 0;
  if (f16) {
#pragma unroll
    for (int j = 0; j < NP; ++j)
      if (tok[j] >= 0) xv[j] = piece_to_f16(xv[j], e[tok[j]]);
  }
  return f16;
}

// Lane (g, i) holds the sums of tokens 4 g + v: their inverse fp16 factors (rows past M carry
// token M - 1's X, and take its factor).
__device__ __forceinline__ f32x4 token_unscale(const int* e, int g, int M) {
  return f32x4{f16_unscale(e[min(4 * g, M - 1)]), f16_unscale(e[min(4 * g + 1, M - 1)]),
               f16_unscale(e[min(4 * g + 2, M - 1)]), f16_unscale(e[min(4 * g + 3, M - 1)])};
}

// A weight's tensor scales (one per segment), read once per workgroup. A walking kernel must not
// read them inside its walk: the epilogue consumes such a load only under a lane mask, which leaves
// the compiler's wait counters unsure of it and makes it wait for every load in flight (the row
// tiles prefetched two ahead) at the next reuse of the register.
static_assert(ATTNQ_MAX_SEGMENTS == 4, "load_tensor_scales holds four segments");
__device__ __forceinline__ f32x4 load_tensor_scales(const float* __restrict__ ts, int n_seg) {
  return f32x4{ts[0], n_seg > 1 ? ts[1] : 0.0f, n_seg > 2 ? ts[2] : 0.0f, n_seg > 3 ? ts[3] : 0.0f};
}

__device__ __forceinline__ float pick_scale(const f32x4& t, int s) { return s == 0 ? t.x : s == 1 ? t.y : s == 2 ? t.z : t.w; }

// One MFMA of the staged-X kernels: X piece xa times 8 codes of word w with block scale s.
template <bool F16>
__device__ __forceinline__ f32x4 mfma_staged(u32x4 xa, uint32_t w, float s, f16x2 s2, f32x4 acc) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(xa), decode8_f16(w, s2), acc, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa), decode8_scaled(w, s), acc, 0, 0, 0);
}

// Tokens-as-rows variant for 4 < M <= 16: A[i][8 g + e] = X[token i][pos] (tokens >= M read as
// zero), B = codes times their block scale in bf16 (exact, see decode8_scaled). All MFMAs of a
// row tile accumulate into one 16 x 16 tile, D[4 g + v][i] = token 4 g + v, weight row i. Lane
// (g, i) needs one scale byte per MFMA pair h: block 2 g + h % 2 + 8 (h / 2), i.e. the row's
// superchunk scale bytes 2 g, 2 g + 1, 2 g + 8 and 2 g + 9.
template <int RT>
__global__ __launch_bounds__(64 * kMaxWaves) void k_gemm_small_m_scaled(const uint8_t* __restrict__ codes,
                                                                       const uint8_t* __restrict__ scales,
                                                                       const float* __restrict__ tensor_scale,
                                                                       SegTable segs, const uint16_t* __restrict__ X,
                                                                       int M, int ldx, float* __restrict__ Y, int ldy,
                                                                       int N, int K, int per) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, ks = blockDim.x >> 6;
  const int g = lane >> 4, i = lane & 15;
  const int row0 = blockIdx.x * (16 * RT);
  const size_t code_pitch = (size_t)K >> 1, scale_pitch = (size_t)K >> 4;

  const uint8_t* crow[RT];
  const uint8_t* srow[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int row = min(row0 + 16 * t + i, N - 1);
    crow[t] = codes + (size_t)row * code_pitch + 16 * g;
    srow[t] = scales + (size_t)row * scale_pitch;
  }
  const bool act = i < M;
  const uint16_t* xrow = X + (size_t)min(i, M - 1) * ldx;

  f32x4 acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  u32x4 xa[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};

  const int nsc = K / kSuper;
  const int s_begin = wave * per, s_end = min(nsc, s_begin + per);
  auto load_w = [&](u32x4 (&cw)[RT][2], uint32_t (&sw)[RT], int sc) {
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const u32x4* cp = reinterpret_cast<const u32x4*>(crow[t] + (size_t)sc * (kSuper / 2));
      cw[t][0] = __builtin_nontemporal_load(cp);
      cw[t][1] = __builtin_nontemporal_load(cp + 4);
      const uint16_t* sp = reinterpret_cast<const uint16_t*>(srow[t] + (size_t)sc * (kSuper / kBlock) + 2 * g);
      sw[t] = sp[0] | ((uint32_t)sp[4] << 16);               // blocks 2 g, 2 g + 1, 2 g + 8, 2 g + 9
    }
  };
  auto compute = [&](const u32x4 (&cw)[RT][2], const uint32_t (&sw)[RT], int sc) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      if (act) {
        const u32x4* xp = reinterpret_cast<const u32x4*>(xrow + (size_t)sc * kSuper + 32 * g + 16 * (h & 1) + 128 * (h >> 1));
        xa[0] = xp[0];
        xa[1] = xp[1];
      }
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const float s = e4m3_byte(sw[t], h);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[0]), decode8_scaled(word(cw[t][h >> 1], 2 * (h & 1)), s),
                                                         acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[1]),
                                                         decode8_scaled(word(cw[t][h >> 1], 2 * (h & 1) + 1), s),
                                                         acc[t], 0, 0, 0);
      }
    }
  };
  if (s_begin < s_end) {
    u32x4 cwa[RT][2], cwb[RT][2];
    uint32_t swa[RT], swb[RT];
    load_w(cwa, swa, s_begin);
    for (int sc = s_begin; sc < s_end; sc += 2) {
      if (sc + 1 < s_end) load_w(cwb, swb, sc + 1);
      compute(cwa, swa, sc);
      if (sc + 1 < s_end) {
        if (sc + 2 < s_end) load_w(cwa, swa, sc + 2);
        compute(cwb, swb, sc + 1);
      }
    }
  }
  // Tail chunks (K % 256 != 0): lane group g takes dword g of the chunk, block 2 ch + g / 2.
  const int nch = K >> 5;
  for (int ch = nsc * (kSuper / kChunkElems) + wave; ch < nch; ch += ks) {
    u32x4 xt = u32x4{0u, 0u, 0u, 0u};
    if (act) xt = *reinterpret_cast<const u32x4*>(xrow + (size_t)ch * kChunkElems + 8 * g);
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(crow[t] - 16 * g + (size_t)ch * 16 + 4 * g);
      const float s = __builtin_amdgcn_cvt_f32_fp8((int)srow[t][(size_t)ch * 2 + (g >> 1)], 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xt), decode8_scaled(w, s), acc[t], 0, 0, 0);
    }
  }

  __shared__ f32x4 part[kMaxWaves - 1][RT][64];
  if (ks > 1) {
    if (wave > 0) {
#pragma unroll
      for (int t = 0; t < RT; ++t) part[wave - 1][t][lane] = acc[t];
    }
    __syncthreads();
    if (wave != 0) return;
    for (int w = 0; w < ks - 1; ++w)
#pragma unroll
      for (int t = 0; t < RT; ++t) acc[t] += part[w][t][lane];
  }
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int row = row0 + 16 * t + i;
    if (row < N) {
      const float ts = tensor_scale[segment_of(segs, row)];
      const float d[4] = {acc[t].x, acc[t].y, acc[t].z, acc[t].w};
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = 4 * g + v;
        if (m < M) Y[(size_t)m * ldy + row] = d[v] * ts;
      }
    }
  }
}

// One-shot slices (k_gemm_small_m_slices): the weights are read the way the batch-1 kernels read
// them, and a wave-private LDS tile turns them into MFMA operands. Workgroup b takes row group b /
// nslices (WAVES tiles of 16 rows, one per wave) and K slice b % nslices (S steps of 1024 elements).
// Every load of the slice is issued at once: per step and wave, 8 code loads (each half-wave reads
// 512 contiguous bytes of one row) and the matching scale loads, and the workgroup's pieces of the
// slice's X windows (M tokens x 1024 elements each), loaded ahead of the weights and staged in LDS.
// Per step, a wave moves its codes into its tile as [row][512 B] (pitch 528, so the 16 rows of a
// read start in different banks) and its scales transposed to [row][lane group][q] (pitch 80);
// lane (g, i) then reads row i's chunk 4 q + g (16 code bytes, 32 elements) with one 16-byte read,
// and its eight chunks' scales with another. MFMA (q, d) takes, in lane group g, elements
// 32 (4 q + g) + 8 d .. + 7: A = X of token i (tokens as rows; rows past M read token M - 1 and are
// never stored), B = the codes decoded with their E4M3 block scale (exact, decode8_scaled); four
// accumulator chains (one per d) are added at the end. A slice's raw partial sums go to the
// workspace, and a second kernel adds the slices in slice order, applies the tensor scale and stores
// Y; a shape of one slice stores Y directly. (Adding the slices in the same launch, by the last
// workgroup to take a ticket as in the split-K GEMV, measured slower here: the publication's round
// trips hold each workgroup's 72 KB of LDS, which is what limits how many run per compute unit.)
// Nothing that uses a load sits in a branch, and scheduling barriers keep X, then the weights,
// ahead of the staging and everything that waits for a weight behind the barrier: with the X
// staging store guarded, the compiler moved an X load behind the weight loads and the barrier
// waited for all of them (down 5376 x 21504 at M = 4: 20.6 -> 19.8 us; at M = 12 and 16 -1.3 us).
constexpr int kSlStep = 1024;                       // K elements per step
constexpr int kSlCodePitch = kSlStep / 2 + 16;      // bytes per row of a wave's code tile
constexpr int kSlScalePitch = 80;                   // bytes per row of a wave's scale tile (64 used)
constexpr int kSlXPitch = 2 * kSlStep + 16;         // bytes per token row of an X window

template <int MT, int WAVES, int S>
__global__ __launch_bounds__(64 * WAVES) void k_gemm_small_m_slices(const uint8_t* __restrict__ codes,
                                                                    const uint8_t* __restrict__ scales,
                                                                    const float* __restrict__ tensor_scale,
                                                                    SegTable segs, const uint16_t* __restrict__ X,
                                                                    int M, int ldx, float* __restrict__ Y, int ldy,
                                                                    int N, int K, int nslices, float* ws) {
  constexpr int kWinPieces = MT * kSlStep / 8;                             // 16-byte pieces of one X window
  constexpr int kXPieces = S * kWinPieces;
  constexpr int kXPerThread = (kXPieces + 64 * WAVES - 1) / (64 * WAVES);
  constexpr int kRows = 16 * WAVES;
  __shared__ __align__(16) uint8_t ctile[WAVES][16 * kSlCodePitch];
  __shared__ __align__(16) uint8_t stile[WAVES][16 * kSlScalePitch];
  __shared__ __align__(16) uint8_t xwin[S][MT * kSlXPitch];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, i = lane & 15;
  const int half = lane >> 5, c_lane = lane & 31;              // load layout: half-wave row, chunk
  const int rg = blockIdx.x / nslices, sl = blockIdx.x - rg * nslices;
  const int row0 = rg * kRows + 16 * wave;
  const uint32_t code_pitch = (uint32_t)K >> 1, scale_pitch = (uint32_t)K >> 4;
  const int cpr = K >> 5;                                       // 32-element chunks per row
  const int st0 = sl * S;
  const int xi = min(i, M - 1);

  // X windows of the slice first (their latency overlaps the weights'), then every weight load
  u32x4 xv[kXPerThread];
#pragma unroll
  for (int j = 0; j < kXPerThread; ++j) {
    const int p = min((int)threadIdx.x + j * 64 * WAVES, kXPieces - 1);
    const int s = p / kWinPieces, r = p - s * kWinPieces;
    const int m = min(r / (kSlStep / 8), M - 1), e = (st0 + s) * kSlStep + 8 * (r % (kSlStep / 8));
    xv[j] = *reinterpret_cast<const u32x4*>(X + (size_t)m * ldx + min(e, K - 8));
  }
  __builtin_amdgcn_sched_barrier(0);
  uint32_t crow[8], srow[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t row = (uint32_t)min(row0 + 2 * j + half, N - 1);     // rows past N load row N-1, never stored
    crow[j] = row * code_pitch;
    srow[j] = row * scale_pitch;
  }
  u32x4 cv[S][8];
  uint32_t sv[S][8];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int c = min((st0 + s) * 32 + c_lane, cpr - 1);      // clamped; chunks past the row are zeroed below
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      cv[s][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(codes + (crow[j] + 16u * (uint32_t)c)));
      sv[s][j] = *reinterpret_cast<const uint16_t*>(scales + (srow[j] + 2u * (uint32_t)c));
    }
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < kXPerThread; ++j) {
    const int p = (int)threadIdx.x + j * 64 * WAVES;
    const int pc = min(p, kXPieces - 1);
    const int s = pc / kWinPieces, r = pc - s * kWinPieces;
    const int m = r / (kSlStep / 8), e = (st0 + s) * kSlStep + 8 * (r % (kSlStep / 8));
    // pieces past the windows go to the padding of window 0's first row, which is never read
    const int off = p < kXPieces ? m * kSlXPitch + 16 * (r % (kSlStep / 8)) : 2 * kSlStep;
    *reinterpret_cast<u32x4*>(&xwin[p < kXPieces ? s : 0][off]) = (m < M && e < K) ? xv[j] : u32x4{0u, 0u, 0u, 0u};
  }
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);       // nothing that waits for a weight load moves above the barrier

  f32x4 acc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) acc[d] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  uint8_t* ct = ctile[wave];
  uint8_t* st = stile[wave];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    // no branch on the step: a step past the row has no valid chunk, so its codes are stored as
    // zeros and it takes no MFMA (a branch would let the compiler move the weight loads behind the
    // barrier, into the branch that uses them)
    const int step = st0 + s;
    {
      const int nck = min(32, cpr - step * 32);                 // valid chunks in this step (<= 0 past the row)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = 2 * j + half;
        *reinterpret_cast<u32x4*>(ct + row * kSlCodePitch + 16 * c_lane) = c_lane < nck ? cv[s][j] : u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<uint16_t*>(st + row * kSlScalePitch + 16 * (c_lane & 3) + 2 * (c_lane >> 2)) = (uint16_t)sv[s][j];
      }
      const u32x4 sc = *reinterpret_cast<const u32x4*>(st + i * kSlScalePitch + 16 * g);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (4 * q < nck) {
          const u32x4 cw = *reinterpret_cast<const u32x4*>(ct + i * kSlCodePitch + 16 * (4 * q + g));
          const uint8_t* xp = &xwin[s][xi * kSlXPitch + 64 * (4 * q + g)];
          const uint32_t sb = word(sc, q >> 1) >> (16 * (q & 1));        // the chunk's two block scales
          const float s0 = __builtin_amdgcn_cvt_f32_fp8((int)sb, 0), s1 = __builtin_amdgcn_cvt_f32_fp8((int)sb, 1);
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const u32x4 xa = *reinterpret_cast<const u32x4*>(xp + 16 * d);
            acc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa), decode8_scaled(word(cw, d), d < 2 ? s0 : s1),
                                                             acc[d], 0, 0, 0);
          }
        }
      }
    }
  }
  const f32x4 a4 = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  const float a[4] = {a4.x, a4.y, a4.z, a4.w};
  // lane (g, i): tokens 4 g + v of weight row row0 + i
  const int row = row0 + i;
  if (nslices == 1) {
    if (row < N) {
      const float ts = tensor_scale[segment_of(segs, row)];
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (4 * g + v < M) Y[(size_t)(4 * g + v) * ldy + row] = a[v] * ts;
    }
    return;
  }
  // the slice's raw partial sums: part[row group][slice][token][row of the group]
  float* part = reinterpret_cast<float*>(ws) + (size_t)rg * nslices * M * kRows + 16 * wave + i;
#pragma unroll
  for (int v = 0; v < 4; ++v)
    if (4 * g + v < M) part[((size_t)sl * M + 4 * g + v) * kRows] = a[v];
}

// Second kernel of a sliced product (stream order makes the partials visible): thread (m, row) adds
// the row group's slices in slice order, applies the tensor scale and stores Y[m][row].
template <int NS>
__global__ __launch_bounds__(256) void k_gemm_small_m_slices_sum(const float* __restrict__ part,
                                                                 const float* __restrict__ tensor_scale, SegTable segs,
                                                                 float* __restrict__ Y, int ldy, int M, int N,
                                                                 int nslices) {
  const int row = blockIdx.x * 256 + threadIdx.x, m = blockIdx.y;
  if (row >= N) return;
  const int rg = row >> 6, r = row & 63;
  const float* p = part + ((size_t)rg * nslices * M + m) * 64 + r;
  const float ts = tensor_scale[segment_of(segs, row)];
  const size_t step = (size_t)M * 64;
  // NS slices' loads in flight at once (8 or 32, the launcher's choice by the slice count), then
  // added in slice order
  float t = 0.0f;
  for (int k0 = 0; k0 < nslices; k0 += NS) {
    float a[NS];
#pragma unroll
    for (int k = 0; k < NS; ++k)
      if (k0 + k < nslices) a[k] = p[(size_t)(k0 + k) * step];
#pragma unroll
    for (int k = 0; k < NS; ++k)
      if (k0 + k < nslices) t += a[k];
  }
  Y[(size_t)m * ldy + row] = t * ts;
}

void launch_slices_sum(const float* part, const float* tensor_scale, const SegTable& t, float* Y, int ldy, int M, int N,
                       int nslices, hipStream_t stream) {
  const dim3 grid((unsigned)((N + 255) / 256), (unsigned)M);
  if (nslices <= 8)
    k_gemm_small_m_slices_sum<8><<<grid, 256, 0, stream>>>(part, tensor_scale, t, Y, ldy, M, N, nslices);
  else
    k_gemm_small_m_slices_sum<32><<<grid, 256, 0, stream>>>(part, tensor_scale, t, Y, ldy, M, N, nslices);
}

// Walking K strips (k_gemm_small_m_walk): a workgroup of four waves owns one strip of SC chunks
// (32 SC elements) of K and walks the row groups (64 rows, 16 per wave) with a fixed stride; the
// grid is what the device holds at once, so there is no second round. The strip's X (tokens up to
// MT) is staged in LDS once, in fp16 when the window allows it (stage_f16). Each wave keeps the
// codes and scales of its next two row tiles in flight in two register sets while it turns the
// current tile into MFMA operands through its LDS tile, with the slices' operand placement. A
// strip's raw partial sums go to the workspace in the slices' layout and k_gemm_small_m_slices_sum
// adds them in strip order; a single strip stores Y directly. Strips are whole (SC divides the
// row's chunks) and 128-byte aligned (SC a multiple of 8), so every cache line of codes is read by
// one strip.
//
// Loads go through buffer resources bounded to the codes' and scales' extents: a load at an offset
// past the end returns zeros without a memory request (the bounds check covers the whole offset,
// kept in the VGPR operand). Rows past N and the tiles past the end of a walk (row0 = N) read
// zeros that way, and so do the lanes with nothing to load, so every lane loads and nothing here
// branches or clamps: the number of loads in flight is then the same on every path through the
// walk, which lets the compiler's wait counts leave the tiles loaded ahead in flight. (The
// launcher keeps (N + 16) K below 2^32, so no offset wraps.)
template <int SC>
struct WalkIn {
  u32x4 cv[8];          // code chunk of rows 2 j + half (one 16-byte chunk per lane)
  u32x4 sv;             // 8 chunks' scale pairs: row lane / (SC / 8), chunks 8 (lane % (SC / 8)) ..
};

struct WalkRes {
  __amdgpu_buffer_rsrc_t codes, scales;
};

constexpr int kBufNontemporal = 2;        // buffer load cache policy: nt
constexpr uint32_t kBufOff = 0x80000000u;  // a column offset past any extent

// ccol / scol: the lane's byte offset in a code / scale row (kBufOff for lanes with nothing to load).
template <int SC>
__device__ __forceinline__ void walk_loads(WalkIn<SC>& in, const WalkRes& res, int row0, int half, uint32_t ccol,
                                           int srow, uint32_t scol, uint32_t code_pitch, uint32_t scale_pitch) {
  const uint32_t co = (uint32_t)(row0 + half) * code_pitch + ccol;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    in.cv[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(res.codes, (int)(co + 2u * j * code_pitch),
                                                                               0, kBufNontemporal));
  in.sv = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                        res.scales, (int)((uint32_t)(row0 + srow) * scale_pitch + scol), 0, 0));
}

// One row tile's MFMAs over the strip (codes and scales in the wave's LDS tile, X at xrow), with
// fp16 or bf16 operands.
template <int SC, bool F16>
__device__ __forceinline__ f32x4 strip_mfma(const uint8_t* __restrict__ ct, const uint8_t* __restrict__ xrow,
                                            const u32x4& sc, int g, int i) {
  constexpr int kCodePitch = SC * 16 + 16;
  f32x4 acc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) acc[d] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int q = 0; q < SC / 4; ++q) {
    const u32x4 cw = *reinterpret_cast<const u32x4*>(ct + i * kCodePitch + 16 * (4 * q + g));
    const uint8_t* xp = xrow + 64 * (4 * q + g);
    const uint32_t sw = word(sc, q >> 1);                             // chunks 4 q + g, 4 q + 4 + g: 2 scales each
    float s0 = 0.0f, s1 = 0.0f;
    f16x2 h0 = {}, h1 = {};
    if constexpr (F16) {
      const f16x2 h = (q & 1) ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, true)
                              : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, false);
      h0 = f16x2{h.x, h.x};
      h1 = f16x2{h.y, h.y};
    } else {
      const uint32_t sb = sw >> (16 * (q & 1));
      s0 = __builtin_amdgcn_cvt_f32_fp8((int)sb, 0);
      s1 = __builtin_amdgcn_cvt_f32_fp8((int)sb, 1);
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const u32x4 xa = *reinterpret_cast<const u32x4*>(xp + 16 * d);
      acc[d] = mfma_staged<F16>(xa, word(cw, d), d < 2 ? s0 : s1, d < 2 ? h0 : h1, acc[d]);
    }
  }
  return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

template <int MT, int SC>
__device__ __forceinline__ void walk_tile(WalkIn<SC>& in, uint8_t* __restrict__ ct, uint8_t* __restrict__ st,
                                          const uint8_t* __restrict__ xwin, const WalkRes& res, const f32x4& tsv,
                                          const SegTable& segs, float* __restrict__ Y, int ldy, int M, int N, int rg,
                                          int ahead_rg, int groups, int wave, int lane, uint32_t ccol, int srow,
                                          uint32_t scol, int sl, int nstrips, uint32_t code_pitch, uint32_t scale_pitch,
                                          float* ws, bool f16, f32x4 unscale) {
  constexpr int kCodePitch = SC * 16 + 16;
  constexpr int kXPitch = SC * 64 + 16;
  constexpr int kPieces = SC / 8;
  const int g = lane >> 4, i = lane & 15, half = lane >> 5, c_lane = lane & 31;
  // This tile's codes and scales into the wave's LDS tile, then the registers take the tile two
  // ahead. Lanes past the strip's width write their row's padding slot. The scale tile is
  // [row][16 (c % 4) + 2 (c / 4)] (pitch 80): the lane's 8 chunks 8 p + k go out as four dwords
  // (chunks k and k + 4 side by side); lanes without a piece write the spare row 16.
#pragma unroll
  for (int j = 0; j < 8; ++j)
    *reinterpret_cast<u32x4*>(ct + (2 * j + half) * kCodePitch + 16 * min(c_lane, SC)) = in.cv[j];
  {
    const int p = lane % kPieces, r = lane < 16 * kPieces ? lane / kPieces : 16;
    uint8_t* d = st + r * kSlScalePitch + 4 * p;
    const uint32_t d0 = in.sv.x, d1 = in.sv.y, d2 = in.sv.z, d3 = in.sv.w;
    *reinterpret_cast<uint32_t*>(d) = (d0 & 0xFFFFu) | (d2 << 16);
    *reinterpret_cast<uint32_t*>(d + 16) = (d0 >> 16) | (d2 & 0xFFFF0000u);
    *reinterpret_cast<uint32_t*>(d + 32) = (d1 & 0xFFFFu) | (d3 << 16);
    *reinterpret_cast<uint32_t*>(d + 48) = (d1 >> 16) | (d3 & 0xFFFF0000u);
  }
  walk_loads<SC>(in, res, ahead_rg < groups ? ahead_rg * 64 + 16 * wave : N, half, ccol, srow, scol, code_pitch,
                 scale_pitch);
  // The X operands are the same for every row tile: left visible, the compiler hoists their LDS
  // reads out of the walk and holds all of them in registers, which costs a wave per SIMD. The
  // empty asm makes the offset opaque, so they are read per tile.
  int xoff = min(i, M - 1) * kXPitch;
  asm volatile("" : "+v"(xoff));
  const u32x4 sc = *reinterpret_cast<const u32x4*>(st + i * kSlScalePitch + 16 * g);
  // the window's operand type is uniform: one branch per tile
  const f32x4 a4 = f16 ? strip_mfma<SC, true>(ct, xwin + xoff, sc, g, i) * unscale
                       : strip_mfma<SC, false>(ct, xwin + xoff, sc, g, i);
  const float a[4] = {a4.x, a4.y, a4.z, a4.w};
  const int row = rg * 64 + 16 * wave + i;            // lane (g, i): tokens 4 g + v of this row
  if (nstrips == 1) {
    if (row < N) {
      const float ts = pick_scale(tsv, segment_of(segs, row));
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (4 * g + v < M) Y[(size_t)(4 * g + v) * ldy + row] = a[v] * ts;
    }
    return;
  }
  // [row group][strip][token][64 rows]. The stores are unconditional, for the same reason as the
  // loads: a token row past M read token M - 1's X (and takes its fp16 factor), so its sum is the
  // same value, written to token M - 1's slot.
  float* part = ws + (size_t)rg * nstrips * M * 64 + 16 * wave + i;
#pragma unroll
  for (int v = 0; v < 4; ++v) part[((size_t)sl * M + min(4 * g + v, M - 1)) * 64] = a[v];
}

// The walk proper: row tiles rg, rg + walkers, ... alternately from register sets A and B, as a
// counted loop of two tiles and one tile after it. (With exits between the two tiles, the
// compiler's control flow lets a B tile follow a B tile, and its wait counts then take the A set's
// loads as not in flight and wait for them too.)
template <int MT, int SC>
__device__ __forceinline__ void walk_rows(WalkIn<SC>& A, WalkIn<SC>& B, uint8_t* __restrict__ ct,
                                          uint8_t* __restrict__ st, const uint8_t* __restrict__ xwin,
                                          const WalkRes& res, const f32x4& tsv, const SegTable& segs,
                                          float* __restrict__ Y, int ldy, int M, int N, int rg, int walkers, int groups,
                                          int wave, int lane, uint32_t ccol, int srow, uint32_t scol, int sl,
                                          int nstrips, uint32_t code_pitch, uint32_t scale_pitch, float* ws,
                                          bool f16, f32x4 unscale) {
  const int n = (groups - rg + walkers - 1) / walkers;
  int k = 0;
  for (; k + 1 < n; k += 2) {
    walk_tile<MT, SC>(A, ct, st, xwin, res, tsv, segs, Y, ldy, M, N, rg, rg + 2 * walkers, groups, wave, lane,
                           ccol, srow, scol, sl, nstrips, code_pitch, scale_pitch, ws, f16, unscale);
    rg += walkers;
    walk_tile<MT, SC>(B, ct, st, xwin, res, tsv, segs, Y, ldy, M, N, rg, rg + 2 * walkers, groups, wave, lane,
                           ccol, srow, scol, sl, nstrips, code_pitch, scale_pitch, ws, f16, unscale);
    rg += walkers;
  }
  if (k < n)
    walk_tile<MT, SC>(A, ct, st, xwin, res, tsv, segs, Y, ldy, M, N, rg, rg + 2 * walkers, groups, wave, lane,
                           ccol, srow, scol, sl, nstrips, code_pitch, scale_pitch, ws, f16, unscale);
}

template <int MT, int SC>
__global__ __launch_bounds__(256) void k_gemm_small_m_walk(const uint8_t* __restrict__ codes,
                                                           const uint8_t* __restrict__ scales,
                                                           const float* __restrict__ tensor_scale, SegTable segs,
                                                           const uint16_t* __restrict__ X, int M, int ldx,
                                                           float* __restrict__ Y, int ldy, int N, int K, int nstrips,
                                                           int walkers, float* ws) {
  static_assert(SC % 8 == 0 && SC <= 32, "strips of whole 128-byte lines, at most 32 chunks");
  constexpr int kCodePitch = SC * 16 + 16;
  constexpr int kXPitch = SC * 64 + 16;
  constexpr int kXPieces = MT * SC * 4;                        // 16-byte pieces of the strip's X
  constexpr int kXPerThread = (kXPieces + 255) / 256;
  constexpr int kPieces = SC / 8;                              // 16-byte scale pieces per row
  __shared__ __align__(16) uint8_t ctile[4][16 * kCodePitch];
  __shared__ __align__(16) uint8_t stile[4][17 * kSlScalePitch];
  __shared__ __align__(16) uint8_t xwin[MT * kXPitch];
  __shared__ int xexp[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, c_lane = lane & 31;
  // Workgroups are dealt to the 8 XCDs round-robin; when the grid is a multiple of 8, XCD x takes
  // the x-th eighth of the logical order, so the strips of a row group share one L2 (the scale
  // lines, read 2 SC bytes per strip, are then fetched once).
  const int b = gridDim.x % 8 == 0 ? (int)(blockIdx.x % 8) * (int)(gridDim.x / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
  const int sl = b % nstrips;
  int rg = b / nstrips;                                        // < groups: walkers <= groups
  const int groups = (N + 63) >> 6;
  const int c0 = sl * SC;
  const uint32_t code_pitch = (uint32_t)K >> 1, scale_pitch = (uint32_t)K >> 4;
  const uint32_t ccol = c_lane < SC ? 16u * (uint32_t)(c0 + c_lane) : kBufOff;
  const int srow = lane < 16 * kPieces ? lane / kPieces : 0;
  const uint32_t scol = lane < 16 * kPieces ? 2u * (uint32_t)c0 + 16u * (uint32_t)(lane % kPieces) : kBufOff;
  const f32x4 tsv = load_tensor_scales(tensor_scale, segs.n_seg);
  const WalkRes res{__builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(codes), (short)0, (int)((uint32_t)N * code_pitch),
                                                      0x00020000),
                    __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(scales), (short)0, (int)((uint32_t)N * scale_pitch),
                                                      0x00020000)};

  // the strip's X, then the first two row tiles' weights (all in flight together); X is checked for
  // the fp16 operands and stored to LDS while the weights arrive (the barriers wait for LDS only)
  u32x4 xv[kXPerThread];
  int tok[kXPerThread];
#pragma unroll
  for (int j = 0; j < kXPerThread; ++j) {
    const int pu = (int)threadIdx.x + 256 * j, p = min(pu, kXPieces - 1);
    const int m = p / (SC * 4), r = p - m * (SC * 4);
    const int ch = c0 + (r >> 2);
    const bool ok = m < M;
    xv[j] = ok ? *reinterpret_cast<const u32x4*>(X + (size_t)m * ldx + ch * 32 + 8 * (r & 3)) : u32x4{0u, 0u, 0u, 0u};
    tok[j] = (ok && pu < kXPieces) ? m : -1;
  }
  // (the scheduling barriers keep the two sets' loads in order: a set's last load moved behind the
  // other set's makes the walk's first wait cover both)
  WalkIn<SC> A, B;
  __builtin_amdgcn_sched_barrier(0);
  walk_loads<SC>(A, res, rg * 64 + 16 * wave, half, ccol, srow, scol, code_pitch, scale_pitch);
  __builtin_amdgcn_sched_barrier(0);
  walk_loads<SC>(B, res, rg + walkers < groups ? (rg + walkers) * 64 + 16 * wave : N, half, ccol, srow, scol,
                 code_pitch, scale_pitch);
  __builtin_amdgcn_sched_barrier(0);
  const bool f16 = stage_f16(xv, tok, xexp);
#pragma unroll
  for (int j = 0; j < kXPerThread; ++j) {
    const int p = (int)threadIdx.x + 256 * j;
    if (p < kXPieces) {
      const int m = p / (SC * 4), r = p - m * (SC * 4);
      *reinterpret_cast<u32x4*>(xwin + m * kXPitch + 64 * (r >> 2) + 16 * (r & 3)) = xv[j];
    }
  }
  __syncthreads();
  const f32x4 unscale = f16 ? token_unscale(xexp, lane >> 4, M) : f32x4{1.0f, 1.0f, 1.0f, 1.0f};
  walk_rows<MT, SC>(A, B, ctile[wave], stile[wave], xwin, res, tsv, segs, Y, ldy, M, N, rg, walkers, groups, wave, lane,
                    ccol, srow, scol, sl, nstrips, code_pitch, scale_pitch, ws, f16, unscale);
}

template <int RT>
void launch_scaled(const attnq_nvfp4& W, const uint16_t* X, int M, int ldx, float* Y, int ldy, int ks,
                   hipStream_t stream) {
  SegTable t;
  t.n_seg = W.n_seg;
  for (int s = 0; s < ATTNQ_MAX_SEGMENTS; ++s) t.end[s] = (s < W.n_seg) ? W.seg_end[s] : W.N;
  const int nsc = W.K / kSuper;
  const int per = (nsc + ks - 1) / ks;
  const unsigned grid = (unsigned)((W.N + 16 * RT - 1) / (16 * RT));
  k_gemm_small_m_scaled<RT><<<grid, 64 * ks, 0, stream>>>(W.codes, W.scales, W.tensor_scale, t, X, M, ldx, Y, ldy,
                                                          W.N, W.K, per);
}

template <int RT, int P>
void launch_mfma(const attnq_nvfp4& W, const uint16_t* X, int M, int ldx, float* Y, int ldy, int ks,
                 hipStream_t stream) {
  SegTable t;
  t.n_seg = W.n_seg;
  for (int s = 0; s < ATTNQ_MAX_SEGMENTS; ++s) t.end[s] = (s < W.n_seg) ? W.seg_end[s] : W.N;
  const int nsc = W.K / kSuper;
  const int per = (nsc + ks - 1) / ks;           // superchunks per wave (0 when K < 256)
  const unsigned grid = (unsigned)((W.N + 16 * RT - 1) / (16 * RT));
  k_gemm_small_m_mfma<RT, P><<<grid, 64 * ks, 0, stream>>>(W.codes, W.scales, W.tensor_scale, t, X, M, ldx, Y, ldy,
                                                           W.N, W.K, per);
}

// Launch plan of the one-shot slices: rows of more than 6144 elements, and weights of at least 16384
// rows at M > 4; 4 waves (64 rows) per workgroup and slices of one step (two for 4 < M <= 8 on
// weights of at least 16384 rows). Measured per launch over 8 distinct 31B-like layers in graph
// replays, slices and their sum kernel against the older kernels: at M = 8 down 26.5 against
// 39.9 us, gate|up 45.7 against 58.2, but q|k|v 14.3 against 12.8 and o 11.0 against 10.1 (which
// keep the older kernels); at M = 16 down 27.8 against 47.6 and gate|up 51.9 against 68.2; at M = 4
// down 23.0 against 29.6 (the other projections stay on the batch-1 walk). Workgroups of 2 or 8
// waves and slices of 3 steps measured slower in a timing copy.
struct SlicePlan {
  int mt, s, nslices, groups;
};

bool slice_plan(const attnq_nvfp4& W, int M, SlicePlan* p) {
  if (M < 1 || M > 16 || (W.K <= 6144 && (M <= 4 || W.N < 16384))) return false;
  p->mt = M <= 4 ? 4 : (M <= 8 ? 8 : 16);
  p->s = (p->mt == 8 && W.N >= 16384) ? 2 : 1;
  const int nsteps = (W.K / 32 + 31) / 32;
  p->nslices = (nsteps + p->s - 1) / p->s;
  p->groups = (W.N + 63) / 64;
  return true;
}

template <int MT, int S>
void launch_slices_t(const attnq_nvfp4& W, const uint16_t* X, int M, int ldx, float* Y, int ldy, const SlicePlan& p,
                     float* ws, hipStream_t stream) {
  SegTable t;
  t.n_seg = W.n_seg;
  for (int s = 0; s < ATTNQ_MAX_SEGMENTS; ++s) t.end[s] = (s < W.n_seg) ? W.seg_end[s] : W.N;
  k_gemm_small_m_slices<MT, 4, S><<<(unsigned)(p.groups * p.nslices), 256, 0, stream>>>(
      W.codes, W.scales, W.tensor_scale, t, X, M, ldx, Y, ldy, W.N, W.K, p.nslices, ws);
  if (p.nslices > 1)
    launch_slices_sum(ws, W.tensor_scale, t, Y, ldy, M, W.N, p.nslices, stream);
}

// K split: 12 waves per workgroup (at most one per superchunk). Timed on MI355X over the
// 31B-like layer shapes at M = 4, 8, 16 and row tiles of 1, 2, 4: two 16-row tiles per wave and
// 12 waves are within 5% of the best configuration for every shape.
int pick_ks(const attnq_nvfp4& W) { return max(1, min(12, W.K / kSuper)); }

// Launch plan of the walking strips: rows of more than 6144 elements, and weights of at least 16384
// rows at M > 2, whose rows split into whole strips of 32, 24 or 16 chunks (K = 5376: 7 strips of
// 24; 16384: 16 of 32); tokens padded to 4, 8 or 16 in the X strip. Measured on the 31B-like
// gate|up (43008 x 5376, 8 distinct weights in graph replays, the sum kernel included): M = 3
// 31.8 us and M = 4 33.1 us against 33.4 and 39.3 for the batch-1 walk; at M = 2 the batch-1
// walk stays (30.0 against 31.1).
struct WalkPlan {
  int mt, sc, nstrips, groups;
};

bool walk_plan(const attnq_nvfp4& W, int M, WalkPlan* p) {
  if (M < 1 || M > 16 || (W.K <= 6144 && (M <= 2 || W.N < 16384))) return false;
  if ((int64_t)(W.N + 16) * W.K >= ((int64_t)1 << 32)) return false;    // 32-bit buffer offsets with room for kBufOff
  const int cpr = W.K / 32;
  p->sc = cpr % 32 == 0 ? 32 : (cpr % 24 == 0 ? 24 : (cpr % 16 == 0 ? 16 : 0));
  if (p->sc == 0) return false;                                         // strips must be whole
  p->mt = M <= 4 ? 4 : (M <= 8 ? 8 : 16);
  p->nstrips = cpr / p->sc;
  p->groups = (W.N + 63) / 64;
  return true;
}

template <int MT, int SC>
void launch_walk_t(const attnq_nvfp4& W, const uint16_t* X, int M, int ldx, float* Y, int ldy, const WalkPlan& p,
                   float* ws, hipStream_t stream) {
  static std::atomic<int> cap[64];
  SegTable t;
  t.n_seg = W.n_seg;
  for (int s = 0; s < ATTNQ_MAX_SEGMENTS; ++s) t.end[s] = (s < W.n_seg) ? W.seg_end[s] : W.N;
  int dev = 0, c = 0;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64) c = cap[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_gemm_small_m_walk<MT, SC>, 256, 0) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && per_cu > 0 && cus > 0) {
      c = per_cu * cus;
      if (dev >= 0 && dev < 64) cap[dev].store(c, std::memory_order_relaxed);
    } else {
      c = 512;
    }
  }
  int walkers = max(1, min(p.groups, c / p.nstrips));
  for (int d = 0; d < 7 && walkers > 8 && (walkers * p.nstrips) % 8 != 0; ++d) --walkers;   // a grid of whole eighths
  k_gemm_small_m_walk<MT, SC><<<(unsigned)(p.nstrips * walkers), 256, 0, stream>>>(
      W.codes, W.scales, W.tensor_scale, t, X, M, ldx, Y, ldy, W.N, W.K, p.nstrips, walkers, ws);
  if (p.nstrips > 1)
    launch_slices_sum(ws, W.tensor_scale, t, Y, ldy, M, W.N, p.nstrips, stream);
}

template <int MT>
void launch_walk_mt(const attnq_nvfp4& W, const uint16_t* X, int M, int ldx, float* Y, int ldy, const WalkPlan& p,
                    float* ws, hipStream_t stream) {
  if (p.sc == 24) launch_walk_t<MT, 24>(W, X, M, ldx, Y, ldy, p, ws, stream);
  else if (p.sc == 32) launch_walk_t<MT, 32>(W, X, M, ldx, Y, ldy, p, ws, stream);
  else launch_walk_t<MT, 16>(W, X, M, ldx, Y, ldy, p, ws, stream);
}

// The walking strips take weights of at least 16384 rows (gate|up-like: 43008 x 5376, 34.0 against
// 45.5 us for the slices at M = 8, sum kernel included) and, at 4 < M <= 8, narrower weights with
// long rows (down 5376 x 21504: 22.1 against 24.3 us at M = 8); at M <= 4 and M > 8 those stay on
// the one-shot slices (down 21.0 against 21.2 at M = 4, 24.8 against 25.5 at M = 16).
bool takes_walk(const attnq_nvfp4& W, int M) { return W.N >= 16384 || (M > 4 && M <= 8); }

}  // namespace

int64_t gemm_small_m_splitk_workspace_bytes(int N, int K, int M) {
  attnq_nvfp4 W{};
  W.N = N;
  W.K = K;
  if (N == 0) return 0;
  WalkPlan wp;
  if (takes_walk(W, M) && walk_plan(W, M, &wp)) return wp.nstrips == 1 ? 0 : (int64_t)wp.groups * wp.nstrips * M * 64 * 4;
  SlicePlan p;
  if (!slice_plan(W, M, &p) || p.nslices == 1) return 0;
  return (int64_t)p.groups * p.nslices * M * 64 * 4;
}

hipError_t launch_gemm_nvfp4_small_m_splitk(const attnq_nvfp4& W, const uint16_t* X, int M, int ldx, float* Y, int ldy,
                                            void* ws, hipStream_t stream) {
  if (W.N == 0 || M == 0) return hipSuccess;
  float* w = static_cast<float*>(ws);
  WalkPlan wp;
  if (takes_walk(W, M) && walk_plan(W, M, &wp)) {
    if (wp.mt == 4) launch_walk_mt<4>(W, X, M, ldx, Y, ldy, wp, w, stream);
    else if (wp.mt == 8) launch_walk_mt<8>(W, X, M, ldx, Y, ldy, wp, w, stream);
    else launch_walk_mt<16>(W, X, M, ldx, Y, ldy, wp, w, stream);
    return hipGetLastError();
  }
  SlicePlan p;
  if (!slice_plan(W, M, &p)) return launch_gemm_nvfp4_small_m(W, X, M, ldx, Y, ldy, stream);
  if (p.mt == 4) launch_slices_t<4, 1>(W, X, M, ldx, Y, ldy, p, w, stream);
  else if (p.mt == 8 && p.s == 2) launch_slices_t<8, 2>(W, X, M, ldx, Y, ldy, p, w, stream);
  else if (p.mt == 8) launch_slices_t<8, 1>(W, X, M, ldx, Y, ldy, p, w, stream);
  else launch_slices_t<16, 1>(W, X, M, ldx, Y, ldy, p, w, stream);
  return hipGetLastError();
}

hipError_t launch_gemm_nvfp4_small_m(const attnq_nvfp4& W, const uint16_t* X, int M, int ldx, float* Y, int ldy,
                                     hipStream_t stream) {
  if (W.N == 0 || M == 0) return hipSuccess;
  if (launch_gemm_nvfp4_tokens(W, X, M, ldx, Y, ldy, stream)) return hipGetLastError();
  if (M <= 4)
    launch_mfma<2, 1>(W, X, M, ldx, Y, ldy, pick_ks(W), stream);
  else
    launch_scaled<2>(W, X, M, ldx, Y, ldy, pick_ks(W), stream);
  return hipGetLastError();
}

}  // namespace attnq
