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

// K split: 12 waves per workgroup (at most one per superchunk). Timed on MI355X over the
// 31B-like layer shapes at M = 4, 8, 16 and row tiles of 1, 2, 4: two 16-row tiles per wave and
// 12 waves are within 5% of the best configuration for every shape.
int pick_ks(const attnq_nvfp4& W) { return max(1, min(12, W.K / kSuper)); }

}  // namespace

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
