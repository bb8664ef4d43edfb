// Decode GEMVs y = x * W^T: the NVFP4 weight-streaming kernels at batch 1 (plain, with the gate|up
// activation epilogue, with the runtime low-rank epilogue and its partial-sum kernels), the same
// walk for 1 <= M <= 4 tokens (k_gemm_nvfp4_tokens), and the bf16 kernels.
//
// "GPU acceleration", "Where GPU time goes": batch-1 decode is dominated by GEMVs that read
// every weight once, and the block-scaled kernel consumes fp4 directly (no dequant launch).
// "Throughput", "The NVFP4 MLP kernels are the least bandwidth-efficient on the step": the
// B200 kernels reach 47% (NVFP4) and 57-65% (bf16) of HBM peak; the down projection ran
// short of parallelism (42 CTAs on 148 SMs), hence the K split below for long rows.
//
// Mapping (gfx950, wave64): a lane owns one 16-byte code chunk (32 fp4 = two scale blocks) of
// R rows per step, so each wave load instruction covers 1 KiB of one row, fully coalesced;
// the 64 B of x for that chunk are loaded once and reused for the R rows. Decode is
// v_cvt_scalef32_pk_bf16_fp4 (two fp4 -> two bf16, exact, scale 1) feeding v_dot2c_f32_bf16
// into a per-block fp32 partial, which is multiplied by its E4M3 scale once per block. Wave
// partials are reduced with DPP; with a K split, the waves of a workgroup meet in LDS.
#include <mutex>

#include "attnq_device.h"
#include "launch.h"

namespace attnq {

namespace {

// One scale block: 16 fp4 (two dwords of codes) against 16 bf16 of x (eight dwords).
__device__ __forceinline__ float dot16_fp4(uint32_t codes_lo, uint32_t codes_hi, const uint32_t* xw) {
  float p = 0.0f;
  p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes_lo, 1.0f, 0),
                                      as_bf16x2(xw[0]), p, false);
  p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes_lo, 1.0f, 1),
                                      as_bf16x2(xw[1]), p, false);
  p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes_lo, 1.0f, 2),
                                      as_bf16x2(xw[2]), p, false);
  p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes_lo, 1.0f, 3),
                                      as_bf16x2(xw[3]), p, false);
  p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes_hi, 1.0f, 0),
                                      as_bf16x2(xw[4]), p, false);
  p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes_hi, 1.0f, 1),
                                      as_bf16x2(xw[5]), p, false);
  p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes_hi, 1.0f, 2),
                                      as_bf16x2(xw[6]), p, false);
  p = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes_hi, 1.0f, 3),
                                      as_bf16x2(xw[7]), p, false);
  return p;
}

// One 16-byte chunk of one row: two blocks, each partial scaled by its E4M3 scale.
__device__ __forceinline__ float chunk_dot(const u32x4 cv, uint32_t sv, const uint32_t* xw, float acc) {
  const float p0 = dot16_fp4(cv.x, cv.y, xw);
  const float p1 = dot16_fp4(cv.z, cv.w, xw + 8);
  acc = __builtin_fmaf(p0, __builtin_amdgcn_cvt_f32_fp8((int)sv, 0), acc);
  acc = __builtin_fmaf(p1, __builtin_amdgcn_cvt_f32_fp8((int)sv, 1), acc);
  return acc;
}

// Epilogue of the gate|up projection with its activation (the input of down): row pair
// (j, F + j) of a fused [gate; up] weight gives h[j] = bf16(act(gate_j) * up_j), computed in fp32.
__device__ __forceinline__ float activation(float g, int act) {
  if (act == ATTNQ_ACT_GELU_TANH) {
    const float inner = 0.7978845608028654f * (g + 0.044715f * g * g * g);   // sqrt(2/pi)
    return 0.5f * g * (1.0f + tanhf(inner));
  }
  if (act == ATTNQ_ACT_SILU) return g / (1.0f + expf(-g));
  return g;                                                                   // ATTNQ_ACT_IDENTITY
}

__device__ __forceinline__ void store_glu(uint16_t* h, int j, float g, float u, int act) {
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  const bf16x2v p = {(__bf16)(activation(g, act) * u), (__bf16)0.0f};
  h[j] = (uint16_t)(__builtin_bit_cast(uint32_t, p) & 0xFFFFu);
}

// Runtime low-rank epilogue (EPI 2): for a row of segment g,
//   y[row] = s[row] * (x . weight0[row]) + sum_k U[row][k] t[g][k],  t[g] = V[g]^T x.
// The partial-sum kernels leave P partial sums of t per segment (one per 32 KB chunk of V), laid out
// part[g][p][k]. Each wave folds them into its rows directly: with n = P r, lane l takes the
// flat indices i = l, l + 64, ... < n and sums U[row][i mod r] * part[g][i] (a fixed order), and
// the wave adds its lanes. The one-shot kernels load a lane's first two values right after the
// weight loads are issued; there is no LDS and no barrier, so the kernel keeps the plain GEMV's
// shape.
constexpr int kLrThreads = 256;     // threads of the partial-sum kernel
constexpr int kLrChunk = 16384;     // V elements behind one partial (32 KB of bf16)

struct LowRank {
  const uint16_t* s;     // [N] bf16 or null (s = 1)
  const uint16_t* U;     // [N][r] bf16
  const float* part;     // [n_seg][P][r] partial sums of V^T x
  int r, P;
};

// Values loaded ahead of the main loop (PF partials per lane and, when PF > 0 and r divides 64,
// U[row][lane mod r]). They are kept as loaded -- raw bits, converted only at their use after the
// main loop -- and each load is issued unconditionally, from x when its operand is absent, with
// the choice made by a uniform select at the use: no branch and no wait sits between these loads
// and the weight loads issued before them.
template <int R, int PF>
struct LrRegs {
  float pv[PF > 0 ? PF : 1];   // part[g0][min(lane + 64 (ks + KS m), n - 1)]
  uint32_t ub[R];              // U[row][lane mod r] bits of the wave's rows
  uint32_t sb;                 // s bits of the row this lane stores (lane < R)
  int g0;                      // segment of the wave's first row
};

template <int R, int PF, int KS, class RowOf>
__device__ __forceinline__ void lr_prefetch(LrRegs<R, PF>& st, const LowRank& lr, const SegTable& segs,
                                            const RowOf& row_of, int lane, int ks, const void* dummy) {
  st.g0 = segment_of(segs, row_of(0));
  const uint16_t* sp = lr.s != nullptr ? lr.s + row_of(min(lane, R - 1)) : static_cast<const uint16_t*>(dummy);
  st.sb = *sp;
  if constexpr (PF > 0) {
    // distinct dummy addresses (x[m], x[r]; x holds at least 32 elements) keep the compiler from
    // merging the loads of an absent operand into one load plus register copies, which would wait
    const int n = lr.P * lr.r;
    const float* pg = n > 0 ? lr.part + (size_t)st.g0 * n : static_cast<const float*>(dummy);
#pragma unroll
    for (int m = 0; m < PF; ++m) st.pv[m] = pg[n > 0 ? min(lane + 64 * (ks + KS * m), n - 1) : m];
    // U[row][lane mod r] is only used when r divides 64, i.e. r is a power of two (mask, no division)
    const bool fixed_k = lr.r > 0 && 64 % lr.r == 0;
#pragma unroll
    for (int r = 0; r < R; ++r)
      st.ub[r] = *(fixed_k ? lr.U + (size_t)row_of(r) * lr.r + (lane & (lr.r - 1))
                           : static_cast<const uint16_t*>(dummy) + r);
  }
}

// d[r] = sum over the wave's indices i < P r of U[row_r][i mod r] * part[g][i] (g the row's
// segment): lane l of K slice ks (of KS) takes i = l + 64 (ks + KS m), m = 0, 1, ..., in that
// order, then the wave adds its lanes; every lane gets the sums. The KS slices' sums are added
// in slice order by the caller.
template <int R, int PF, int KS, class RowOf>
__device__ __forceinline__ void lr_row_terms(const LrRegs<R, PF>& st, const LowRank& lr, const SegTable& segs,
                                             const RowOf& row_of, int lane, int ks, float* d) {
  const int n = lr.P * lr.r;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = row_of(r);
    const uint16_t* u = lr.U + (size_t)row * lr.r;
    const int g = segment_of(segs, row);
    const float* pg = lr.part + (size_t)g * n;
    float& c = d[r];
    c = 0.0f;
    if (n > 0) {
      if (PF > 0 && g == st.g0 && 64 % lr.r == 0) {
        const float uk = bf16_bits_to_f32((uint16_t)st.ub[r]);
#pragma unroll
        for (int m = 0; m < (PF > 0 ? PF : 1); ++m)
          if (lane + 64 * (ks + KS * m) < n) c = __builtin_fmaf(uk, st.pv[m], c);
        for (int i = lane + 64 * (ks + KS * PF); i < n; i += 64 * KS) c = __builtin_fmaf(uk, pg[i], c);
      } else {
        for (int i = lane + 64 * ks; i < n; i += 64 * KS) c = __builtin_fmaf(bf16_bits_to_f32(u[i % lr.r]), pg[i], c);
      }
    }
  }
  wave_sums<R>(d);
}

__device__ __forceinline__ float lr_finish(float v, float ts, const LowRank& lr, uint32_t s_bits, float d) {
  v *= ts;
  v *= lr.s != nullptr ? bf16_bits_to_f32((uint16_t)s_bits) : 1.0f;
  return v + d;
}

// EPI 0 stores y; EPI 2 stores the low-rank epilogue's y; EPI 1 is the gate|up epilogue: R == 2, the wave's two rows are j and F + j of a
// two-segment weight (F = N / 2) and it stores h[j] (bf16) instead of y.
template <int R, int KSPLIT, int EPI = 0>
__global__ __launch_bounds__(256) void k_gemv_nvfp4(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                                    const float* __restrict__ tensor_scale, SegTable segs,
                                                    const uint16_t* __restrict__ x, float* __restrict__ y, int N, int K,
                                                    uint16_t* __restrict__ h = nullptr, int act = 0, LowRank lr = {}) {
  static_assert(4 % KSPLIT == 0, "K split must divide the 4 waves of a workgroup");
  static_assert(EPI != 1 || (R == 2 && KSPLIT == 1), "the gate|up epilogue takes one row pair per wave");
  constexpr int kRowGroups = 4 / KSPLIT;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rg = wave / KSPLIT, ks = wave % KSPLIT;
  const int row0 = (blockIdx.x * kRowGroups + rg) * R;
  const int F = N >> 1, pj = blockIdx.x * kRowGroups + rg;       // EPI 1: pair index
  auto row_of = [&](int r) { return EPI == 1 ? min(pj, F - 1) + r * F : min(row0 + r, N - 1); };
  const int cpr = K >> 5;
  const int slice = (cpr + KSPLIT - 1) / KSPLIT;
  const int c_begin = ks * slice;
  const int c_end = min(cpr, c_begin + slice);
  const size_t code_pitch = (size_t)K >> 1;
  const size_t scale_pitch = (size_t)K >> 4;

  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0f;

  // 32-bit byte offsets from the (uniform) tensor bases, one row offset per row
  uint32_t crow[R], srow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t row = (uint32_t)row_of(r);        // clamp: rows past N load row N-1, result discarded
    crow[r] = row * (uint32_t)code_pitch;
    srow[r] = row * (uint32_t)scale_pitch;
  }
  for (int c = c_begin + lane; c < c_end; c += 64) {
    const u32x4* xp = reinterpret_cast<const u32x4*>(x) + 4u * (uint32_t)c;
    const u32x4 x0 = xp[0], x1 = xp[1], x2 = xp[2], x3 = xp[3];
    const uint32_t xw[16] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,
                             x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
    u32x4 cv[R];
    uint32_t sv[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      cv[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(codes + (crow[r] + 16u * (uint32_t)c)));
      sv[r] = *reinterpret_cast<const uint16_t*>(scales + (srow[r] + 2u * (uint32_t)c));
    }
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = chunk_dot(cv[r], sv[r], xw, acc[r]);
  }

  // long rows: the low-rank operands are loaded after the main loop, all at once (issued before
  // the loop instead, their latency hidden, the low-rank stream measured the same)
  [[maybe_unused]] LrRegs<R, 4> lrs;
  if constexpr (EPI == 2) lr_prefetch<R, 4, KSPLIT>(lrs, lr, segs, row_of, lane, ks, x);
  wave_sums<R>(acc);
  [[maybe_unused]] float lrd = 0.0f;
  if constexpr (EPI == 2) {
    float d[R];
    lr_row_terms<R, 4, KSPLIT>(lrs, lr, segs, row_of, lane, ks, d);
    lrd = d[0];
#pragma unroll
    for (int r = 1; r < R; ++r) lrd = (lane == r) ? d[r] : lrd;
  }

  if constexpr (EPI == 1) {
    if (lane == 0 && pj < F) store_glu(h, pj, acc[0] * tensor_scale[0], acc[1] * tensor_scale[1], act);
  } else if constexpr (KSPLIT == 1) {
    if (lane < R) {
      float v = acc[0];
#pragma unroll
      for (int r = 1; r < R; ++r) v = (lane == r) ? acc[r] : v;
      const int row = row0 + lane;
      if (row < N) y[row] = EPI == 2 ? lr_finish(v, tensor_scale[segment_of(segs, row)], lr, lrs.sb, lrd)
                                     : v * tensor_scale[segment_of(segs, row)];
    }
  } else {
    __shared__ float part[4][R];
    [[maybe_unused]] __shared__ float partd[EPI == 2 ? 4 : 1][R];
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) part[wave][r] = acc[r];
    }
    if constexpr (EPI == 2) {
      if (lane < R) partd[wave][lane] = lrd;
    }
    __syncthreads();
    if (ks == 0 && lane < R) {
      float v = 0.0f;
#pragma unroll
      for (int s = 0; s < KSPLIT; ++s) v += part[wave + s][lane];
      if constexpr (EPI == 2) {
        lrd = 0.0f;
#pragma unroll
        for (int s = 0; s < KSPLIT; ++s) lrd += partd[wave + s][lane];
      }
      const int row = row0 + lane;
      if (row < N) y[row] = EPI == 2 ? lr_finish(v, tensor_scale[segment_of(segs, row)], lr, lrs.sb, lrd)
                                     : v * tensor_scale[segment_of(segs, row)];
    }
  }
}

// One-shot variant for rows of at most S*64 chunks per wave slice: every wave issues the code
// and scale loads of its whole slice (S steps x R rows) before computing, which keeps the most
// bytes in flight per wave. With XL the workgroup stages x in LDS once, transposed so that the
// four 16-byte quarter reads of a chunk ([q][chunk]) and the staging stores are bank-conflict
// free. XFIRST loads x (at most XI 16-byte pieces per thread) into registers ahead of the weight
// loads; without it, x is loaded after them in a plain loop. Nothing that uses a load may sit in a
// branch: with the staging store of a piece guarded (pieces past x skipped) the compiler moved the
// load of a thread's first piece into the guarded store, behind the weight loads, so the staging
// and the barrier waited for every load of the workgroup; and with the compute step
// guarded by the chunk bound it moved later steps' weight loads behind the barrier. So pieces past
// x are stored to a padding entry, every step computes (lanes past the slice on a clamped chunk,
// their sum discarded by a select), and scheduling barriers keep x, then the weights, ahead of the
// staging: the barrier then waits for x alone and each wave computes as its own loads land (token
// 3.19 -> 3.13 ms).
template <int R, int KSPLIT, int S, bool XL, int WAVES, bool XFIRST = false, int XI = 1, int EPI = 0>
__global__ __launch_bounds__(64 * WAVES) void k_gemv_nvfp4_oneshot(const uint8_t* __restrict__ codes,
                                                                   const uint8_t* __restrict__ scales,
                                                                   const float* __restrict__ tensor_scale, SegTable segs,
                                                                   const uint16_t* __restrict__ x, float* __restrict__ y,
                                                                   int N, int K, uint16_t* __restrict__ h = nullptr,
                                                                   int act = 0, LowRank lr = {}) {
  static_assert(WAVES % KSPLIT == 0, "K split must divide the waves of a workgroup");
  static_assert(!XFIRST || XL, "x-first staging is an LDS staging");
  static_assert(EPI != 1 || (R == 2 && KSPLIT == 1), "the gate|up epilogue takes one row pair per wave");
  // x in LDS as [quarter][chunk] with a compile-time pitch, so the four quarter reads of a chunk
  // use immediate offsets: the longest row the kernel takes (KSPLIT x S x 64 chunks) plus 4
  // entries, which moves each quarter by 64 bytes across the banks. Without the pad the quarters
  // start a multiple of 256 bytes apart, and the staging store, whose four lanes per chunk write
  // the four quarters, is a 4-way bank conflict (SQ_LDS_BANK_CONFLICT); the quarter reads are
  // 1 KiB contiguous per wave either way.
  constexpr int kPitch = KSPLIT * S * 64 + 4;
  __shared__ u32x4 xs[XL ? 4 * kPitch : 1];
  constexpr int kRowGroups = WAVES / KSPLIT;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rg = wave / KSPLIT, ks = wave % KSPLIT;
  const int row0 = (blockIdx.x * kRowGroups + rg) * R;
  const int F = N >> 1, pj = blockIdx.x * kRowGroups + rg;       // EPI 1: pair index
  auto row_of = [&](int r) { return EPI == 1 ? min(pj, F - 1) + r * F : min(row0 + r, N - 1); };
  const int cpr = K >> 5;
  const int slice = (cpr + KSPLIT - 1) / KSPLIT;
  const int c_begin = ks * slice;
  const int c_end = min(cpr, c_begin + slice);
  const size_t code_pitch = (size_t)K >> 1;
  const size_t scale_pitch = (size_t)K >> 4;
  const u32x4* xg = reinterpret_cast<const u32x4*>(x);

  u32x4 xst[XI];
  if constexpr (XFIRST) {
#pragma unroll
    for (int j = 0; j < XI; ++j) xst[j] = xg[min((int)threadIdx.x + j * 64 * WAVES, K / 8 - 1)];
    __builtin_amdgcn_sched_barrier(0);
  }
  // 32-bit byte offsets from the (uniform) tensor bases: one row offset per row, and each load
  // adds only its (clamped) chunk offset
  uint32_t crow[R], srow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t row = (uint32_t)row_of(r);
    crow[r] = row * (uint32_t)(K >> 1);
    srow[r] = row * (uint32_t)(K >> 4);
  }
  u32x4 cv[S][R];
  uint32_t sv[S][R];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const uint32_t c = (uint32_t)min(c_begin + s * 64 + lane, cpr - 1);   // clamped: lanes past the slice reload a valid chunk
#pragma unroll
    for (int r = 0; r < R; ++r) {
      cv[s][r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(codes + (crow[r] + 16u * c)));
      sv[s][r] = *reinterpret_cast<const uint16_t*>(scales + (srow[r] + 2u * c));
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  [[maybe_unused]] LrRegs<R, 2> lrs;
  if constexpr (EPI == 2) lr_prefetch<R, 2, KSPLIT>(lrs, lr, segs, row_of, lane, ks, x);
  if constexpr (XFIRST) {
#pragma unroll
    for (int j = 0; j < XI; ++j) {
      const int i = threadIdx.x + j * 64 * WAVES;
      xs[i < K / 8 ? (i & 3) * kPitch + (i >> 2) : (i & 3) * kPitch + kPitch - 1] = xst[j];
    }
    __syncthreads();
  } else if constexpr (XL) {
    for (int i = threadIdx.x; i < K / 8; i += 64 * WAVES) xs[(i & 3) * kPitch + (i >> 2)] = xg[i];
    __syncthreads();
  }
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0f;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int c = c_begin + s * 64 + lane;
    if constexpr (XL) {
      const u32x4 x0 = xs[c], x1 = xs[kPitch + c], x2 = xs[2 * kPitch + c], x3 = xs[3 * kPitch + c];
      const uint32_t xw[16] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,
                               x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float a = chunk_dot(cv[s][r], sv[s][r], xw, acc[r]);
        acc[r] = c < c_end ? a : acc[r];
      }
      continue;
    }
    if (c < c_end) {
      u32x4 x0, x1, x2, x3;
      if constexpr (XL) {
        x0 = xs[c]; x1 = xs[kPitch + c]; x2 = xs[2 * kPitch + c]; x3 = xs[3 * kPitch + c];
      } else {
        const u32x4* xp = reinterpret_cast<const u32x4*>(x + (size_t)c * kChunkElems);
        x0 = xp[0]; x1 = xp[1]; x2 = xp[2]; x3 = xp[3];
      }
      const uint32_t xw[16] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,
                               x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = chunk_dot(cv[s][r], sv[s][r], xw, acc[r]);
    }
  }
  wave_sums<R>(acc);
  [[maybe_unused]] float lrd = 0.0f;
  if constexpr (EPI == 2) {
    float d[R];
    lr_row_terms<R, 2, KSPLIT>(lrs, lr, segs, row_of, lane, ks, d);
    lrd = d[0];
#pragma unroll
    for (int r = 1; r < R; ++r) lrd = (lane == r) ? d[r] : lrd;
  }
  if constexpr (EPI == 1) {
    if (lane == 0 && pj < F) store_glu(h, pj, acc[0] * tensor_scale[0], acc[1] * tensor_scale[1], act);
  } else if constexpr (KSPLIT == 1) {
    if (lane < R) {
      float v = acc[0];
#pragma unroll
      for (int r = 1; r < R; ++r) v = (lane == r) ? acc[r] : v;
      const int row = row0 + lane;
      if (row < N) y[row] = EPI == 2 ? lr_finish(v, tensor_scale[segment_of(segs, row)], lr, lrs.sb, lrd)
                                     : v * tensor_scale[segment_of(segs, row)];
    }
  } else {
    __shared__ float part[WAVES][R];
    [[maybe_unused]] __shared__ float partd[EPI == 2 ? WAVES : 1][R];
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) part[wave][r] = acc[r];
    }
    if constexpr (EPI == 2) {
      if (lane < R) partd[wave][lane] = lrd;
    }
    __syncthreads();
    if (ks == 0 && lane < R) {
      float v = 0.0f;
#pragma unroll
      for (int k2 = 0; k2 < KSPLIT; ++k2) v += part[wave + k2][lane];
      if constexpr (EPI == 2) {
        lrd = 0.0f;
#pragma unroll
        for (int k2 = 0; k2 < KSPLIT; ++k2) lrd += partd[wave + k2][lane];
      }
      const int row = row0 + lane;
      if (row < N) y[row] = EPI == 2 ? lr_finish(v, tensor_scale[segment_of(segs, row)], lr, lrs.sb, lrd)
                                     : v * tensor_scale[segment_of(segs, row)];
    }
  }
}

// Cross-workgroup K split for long rows (the down projection, 5376 x 21504: rows too few for the
// batch-1 kernels to fill the chip with whole rows). Workgroup b takes row tile b / SK (WAVES x R
// rows, R per wave) and K slice b % SK: it stages its slice of x in LDS and runs the one-shot walk
// over it (every code and scale load of the slice issued at once, x loaded ahead of them, staging and
// compute free of branches as in the one-shot kernel: token 3.124 -> 3.097 ms), then
// writes the tile's raw partial sums into the tile's record. The workgroup that arrives last at the
// tile's ticket adds the SK partials of each row in slice order (so the bits do not depend on the
// arrival order), applies the tensor scale, stores y and returns the ticket to zero. Nothing waits:
// a workgroup either finishes the tile or leaves.
//
// Publication without cache maintenance: an agent-scope release/acquire fence pair writes back and
// invalidates an XCD's whole L2 on this part, and with it the kernel measured 71.5 us instead of
// 14.6 us. So the partials are written and read with agent-scope atomic stores and loads, which go
// through the caches to the coherent level; a workgroup-scope fence plus a wait for the vector-memory
// counter orders the partial stores before the ticket increment, and the same pair after the
// increment keeps the partial loads behind it.
//
// Workspace: one record per row tile at a fixed stride, so that weights of any shape can take
// turns on one workspace: the ticket in the record's first 64-byte slot, then one slot per K slice
// with the tile's 16 partial sums (fp32).
constexpr int kSplitSlotBytes = 64;
constexpr int kSplitMaxSlices = 12;
constexpr int kSplitRecordBytes = kSplitSlotBytes * (1 + kSplitMaxSlices);

__device__ __forceinline__ void wait_vector_memory() {
  __builtin_amdgcn_s_waitcnt(0x0F70);          // vmcnt(0); expcnt and lgkmcnt left at their maxima
}

// EPI 2: the runtime low-rank epilogue of attnq_gemv_nvfp4_lowrank. Slice ks also takes its share of
// the row terms d = sum over i < P r of U[row][i mod r] part[g][i] (i in [ks c, (ks + 1) c), c = ceil(P r
// / SK), lanes stepping by 64, then the wave sum) and publishes it in slot 1 + SK + ks of the record
// (so SK <= 6); the finishing workgroup adds the SK shares in slice order and stores
// y = v ts s + d.
template <int R, int S, int WAVES, int XI, int SK, int EPI = 0>
__global__ __launch_bounds__(64 * WAVES) void k_gemv_nvfp4_splitk(const uint8_t* __restrict__ codes,
                                                                  const uint8_t* __restrict__ scales,
                                                                  const float* __restrict__ tensor_scale, SegTable segs,
                                                                  const uint16_t* __restrict__ x, float* __restrict__ y,
                                                                  int N, int K, uint8_t* ws, LowRank lr = {}) {
  constexpr int kPitch = S * 64 + 4;          // padded as in the one-shot kernel (conflict-free staging)
  constexpr int kTileRows = WAVES * R;
  static_assert(kTileRows * 4 == kSplitSlotBytes && SK <= kSplitMaxSlices, "a slice's partials fill one slot");
  static_assert(EPI == 0 || (EPI == 2 && 2 * SK <= kSplitMaxSlices), "the row-term shares fill the slots after the partials");
  __shared__ u32x4 xs[4 * kPitch];
  __shared__ float red[kTileRows];
  [[maybe_unused]] __shared__ float redd[EPI == 2 ? kTileRows : 1];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tile = blockIdx.x / SK, ks = blockIdx.x - tile * SK;
  const int row0 = tile * kTileRows + wave * R;
  const int cpr = K >> 5;
  const int slice = (cpr + SK - 1) / SK;
  const int c_begin = ks * slice;                       // the launcher guarantees c_begin < cpr
  const int nck = min(cpr, c_begin + slice) - c_begin;  // chunks of this slice, 1 .. S * 64
  const u32x4* xg = reinterpret_cast<const u32x4*>(x) + 4 * c_begin;

  u32x4 xst[XI];
#pragma unroll
  for (int j = 0; j < XI; ++j) xst[j] = xg[min((int)threadIdx.x + j * 64 * WAVES, 4 * nck - 1)];
  __builtin_amdgcn_sched_barrier(0);
  uint32_t crow[R], srow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t row = (uint32_t)min(row0 + r, N - 1);     // rows past N load row N-1, result discarded
    crow[r] = row * (uint32_t)(K >> 1);
    srow[r] = row * (uint32_t)(K >> 4);
  }
  u32x4 cv[S][R];
  uint32_t sv[S][R];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const uint32_t c = (uint32_t)(c_begin + min(s * 64 + lane, nck - 1));   // clamped into the slice
#pragma unroll
    for (int r = 0; r < R; ++r) {
      cv[s][r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(codes + (crow[r] + 16u * c)));
      sv[s][r] = *reinterpret_cast<const uint16_t*>(scales + (srow[r] + 2u * c));
    }
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < XI; ++j) {
    const int i = threadIdx.x + j * 64 * WAVES;
    xs[i < 4 * nck ? (i & 3) * kPitch + (i >> 2) : (i & 3) * kPitch + kPitch - 1] = xst[j];
  }
  __syncthreads();
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0f;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int c = s * 64 + lane;
    const u32x4 x0 = xs[c], x1 = xs[kPitch + c], x2 = xs[2 * kPitch + c], x3 = xs[3 * kPitch + c];
    const uint32_t xw[16] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,
                             x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float a = chunk_dot(cv[s][r], sv[s][r], xw, acc[r]);
      acc[r] = c < nck ? a : acc[r];
    }
  }
  wave_sums<R>(acc);
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) red[wave * R + r] = acc[r];
  }
  if constexpr (EPI == 2) {
    const int n = lr.P * lr.r;
    const int cs = (n + SK - 1) / SK, i_end = min(n, (ks + 1) * cs);
    float d[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int rw = min(row0 + r, N - 1);
      const float* pg = lr.part + (size_t)segment_of(segs, rw) * n;
      const uint16_t* u = lr.U + (size_t)rw * lr.r;
      float c = 0.0f;
      for (int i = ks * cs + lane; i < i_end; i += 64) c = __builtin_fmaf(bf16_bits_to_f32(u[i % lr.r]), pg[i], c);
      d[r] = c;
    }
    wave_sums<R>(d);
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) redd[wave * R + r] = d[r];
    }
  }
  __syncthreads();
  if (wave != 0) return;
  // wave 0 publishes the tile's partials in the tile's record and takes its ticket
  const int row = tile * kTileRows + lane;
  const bool mine = lane < kTileRows && row < N;
  uint32_t* ticket = reinterpret_cast<uint32_t*>(ws + (size_t)tile * kSplitRecordBytes);
  float* part = reinterpret_cast<float*>(ws + (size_t)tile * kSplitRecordBytes + kSplitSlotBytes) + lane;
  if (mine) __hip_atomic_store(part + ks * kTileRows, red[lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if constexpr (EPI == 2) {
    if (mine) __hip_atomic_store(part + (SK + ks) * kTileRows, redd[lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  wait_vector_memory();                                    // the partial stores have completed
  uint32_t arrived = 0u;
  if (lane == 0) arrived = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (__builtin_amdgcn_readfirstlane(arrived) != SK - 1) return;       // lane 0's count, wave-uniform
  wait_vector_memory();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");   // the partial loads stay behind the ticket
  if (mine) {
    float v = __hip_atomic_load(part, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int k2 = 1; k2 < SK; ++k2)
      v += __hip_atomic_load(part + k2 * kTileRows, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if constexpr (EPI == 2) {
      float dd = __hip_atomic_load(part + SK * kTileRows, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int k2 = 1; k2 < SK; ++k2)
        dd += __hip_atomic_load(part + (SK + k2) * kTileRows, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      y[row] = lr_finish(v, tensor_scale[segment_of(segs, row)], lr, lr.s != nullptr ? lr.s[row] : 0u, dd);
    } else {
      y[row] = v * tensor_scale[segment_of(segs, row)];
    }
  }
  if (lane == 0) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(256) void k_clear_words(uint32_t* __restrict__ p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0u;
}

// Small-M product for M = 1 .. 4 tokens on the batch-1 walk (rows of at most S x 64 chunks): the
// weight loads are the one-shot kernel's (each wave load instruction 1 KiB of one row, all of a
// lane's loads issued at once), every token's x is staged in LDS as [token][quarter][chunk], and a
// wave decodes the fp4 chunk of each of its R rows once and takes its dot products with all MT
// tokens. Per block and token the arithmetic is the batch-1 kernel's (dot2 chain, then the E4M3
// scale by one FMA, the tensor scale last), and a row is summed as there (one wave per row, lane l
// on chunks l, l + 64, ..., the same wave reduction; the waves per workgroup do not enter a row's
// sum), so a token's row equals the batch-1 GEMV of that token bit for bit, whatever M is. The x loads come
// first and the staging and compute have no branches, for the reason given at the one-shot kernel
// (pieces past x go to the padding entry, lanes past the row compute on a clamped chunk and a
// select drops their sum).
template <int MT, int R, int S, int WAVES, int XI>
__global__ __launch_bounds__(64 * WAVES) void k_gemm_nvfp4_tokens(const uint8_t* __restrict__ codes,
                                                                  const uint8_t* __restrict__ scales,
                                                                  const float* __restrict__ tensor_scale,
                                                                  SegTable segs, const uint16_t* __restrict__ X,
                                                                  int ldx, float* __restrict__ Y, int ldy, int N,
                                                                  int K) {
  constexpr int kPitch = S * 64 + 4;        // padded as in the batch-1 kernel (conflict-free staging)
  __shared__ u32x4 xs[MT][4 * kPitch];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row0 = (blockIdx.x * WAVES + wave) * R;
  const int cpr = K >> 5;
  const u32x4* xg = reinterpret_cast<const u32x4*>(X);
  const int xrow = ldx >> 3;                       // 16-byte pieces per X row (ldx % 8 == 0)

  u32x4 xst[MT][XI];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < XI; ++j) xst[m][j] = xg[m * xrow + min((int)threadIdx.x + j * 64 * WAVES, K / 8 - 1)];
  __builtin_amdgcn_sched_barrier(0);
  uint32_t crow[R], srow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t row = (uint32_t)min(row0 + r, N - 1);    // rows past N load row N-1, result discarded
    crow[r] = row * (uint32_t)(K >> 1);
    srow[r] = row * (uint32_t)(K >> 4);
  }
  u32x4 cv[S][R];
  uint32_t sv[S][R];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const uint32_t c = (uint32_t)min(s * 64 + lane, cpr - 1);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      cv[s][r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(codes + (crow[r] + 16u * c)));
      sv[s][r] = *reinterpret_cast<const uint16_t*>(scales + (srow[r] + 2u * c));
    }
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < XI; ++j) {
      const int i = threadIdx.x + j * 64 * WAVES;
      xs[m][i < K / 8 ? (i & 3) * kPitch + (i >> 2) : (i & 3) * kPitch + kPitch - 1] = xst[m][j];
    }
  __syncthreads();

  float acc[R * MT];
#pragma unroll
  for (int a = 0; a < R * MT; ++a) acc[a] = 0.0f;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int c = s * 64 + lane;
    {
      uint32_t wd[R][16];                            // the chunk of each row, decoded to bf16 pairs
      float s0[R], s1[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t cw[4] = {cv[s][r].x, cv[s][r].y, cv[s][r].z, cv[s][r].w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          wd[r][4 * d + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[d], 1.0f, 0));
          wd[r][4 * d + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[d], 1.0f, 1));
          wd[r][4 * d + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[d], 1.0f, 2));
          wd[r][4 * d + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[d], 1.0f, 3));
        }
        s0[r] = __builtin_amdgcn_cvt_f32_fp8((int)sv[s][r], 0);
        s1[r] = __builtin_amdgcn_cvt_f32_fp8((int)sv[s][r], 1);
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const u32x4 x0 = xs[m][c], x1 = xs[m][kPitch + c], x2 = xs[m][2 * kPitch + c], x3 = xs[m][3 * kPitch + c];
        const uint32_t xw[16] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,
                                 x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            p0 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(wd[r][q]), as_bf16x2(xw[q]), p0, false);
            p1 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(wd[r][8 + q]), as_bf16x2(xw[8 + q]), p1, false);
          }
          float a = acc[r * MT + m];
          a = __builtin_fmaf(p0, s0[r], a);
          a = __builtin_fmaf(p1, s1[r], a);
          acc[r * MT + m] = c < cpr ? a : acc[r * MT + m];
        }
      }
    }
  }
  wave_sums<R * MT>(acc);
  if (lane < R * MT) {
    float v = acc[0];
#pragma unroll
    for (int a = 1; a < R * MT; ++a) v = (lane == a) ? acc[a] : v;
    const int r = lane / MT, m = lane - r * MT;
    const int row = row0 + r;
    if (row < N) Y[(size_t)m * ldy + row] = v * tensor_scale[segment_of(segs, row)];
  }
}

// bf16 weights: a lane owns one 16-byte chunk (8 bf16) of R rows per step; x chunk reused.
template <int R>
__global__ __launch_bounds__(256) void k_gemv_bf16(const uint16_t* __restrict__ W, const uint16_t* __restrict__ x,
                                                   float* __restrict__ y, int N, int K) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row0 = (blockIdx.x * 4 + wave) * R;
  const int cpr = K >> 3;
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0f;
#pragma unroll 4           // four chunks' loads in flight per row
  for (int c = lane; c < cpr; c += 64) {
    const u32x4 xv = reinterpret_cast<const u32x4*>(x)[c];
    u32x4 wv[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = min(row0 + r, N - 1);
      wv[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(W + (size_t)row * K) + c);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float a = acc[r];
      a = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(wv[r].x), as_bf16x2(xv.x), a, false);
      a = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(wv[r].y), as_bf16x2(xv.y), a, false);
      a = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(wv[r].z), as_bf16x2(xv.z), a, false);
      a = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(wv[r].w), as_bf16x2(xv.w), a, false);
      acc[r] = a;
    }
  }
  wave_sums<R>(acc);
  if (lane < R) {
    float v = acc[0];
#pragma unroll
    for (int r = 1; r < R; ++r) v = (lane == r) ? acc[r] : v;
    const int row = row0 + lane;
    if (row < N) y[row] = v;
  }
}

// bf16 weights, one-shot (rows of at most S x 64 chunks of 8 elements): a wave owns R rows and
// issues every weight and x load of them (S steps) before computing. Every step computes (lanes
// past the row on a clamped chunk, their sum dropped by a select) and a scheduling barrier keeps
// the loads ahead: with the step guarded, the compiler moved the first step's loads into its
// branch, behind all the others, and the wave waited for every load before its first dot product
// (lm_head 389 -> 385 us, the bf16-attention stream -0.02 ms).
template <int R, int S, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void k_gemv_bf16_oneshot(const uint16_t* __restrict__ W,
                                                                  const uint16_t* __restrict__ x,
                                                                  float* __restrict__ y, int N, int K) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row0 = (blockIdx.x * WAVES + wave) * R;
  const int cpr = K >> 3;
  const u32x4* xg = reinterpret_cast<const u32x4*>(x);
  u32x4 xv[S], wv[S][R];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int c = min(s * 64 + lane, cpr - 1);
    xv[s] = xg[c];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = min(row0 + r, N - 1);
      wv[s][r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(W + (size_t)row * K) + c);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0f;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const bool ok = s * 64 + lane < cpr;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float a = acc[r];
      a = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(wv[s][r].x), as_bf16x2(xv[s].x), a, false);
      a = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(wv[s][r].y), as_bf16x2(xv[s].y), a, false);
      a = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(wv[s][r].z), as_bf16x2(xv[s].z), a, false);
      a = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(wv[s][r].w), as_bf16x2(xv[s].w), a, false);
      acc[r] = ok ? a : acc[r];
    }
  }
  wave_sums<R>(acc);
  if (lane < R) {
    float v = acc[0];
#pragma unroll
    for (int r = 1; r < R; ++r) v = (lane == r) ? acc[r] : v;
    const int row = row0 + lane;
    if (row < N) y[row] = v;
  }
}

// part[g][p][k] = sum over the rows j of chunk p of x[j] V[g][j][k] (V [n_seg][K][r] bf16), one
// workgroup per (chunk, segment); a chunk is floor(16384 / r) rows of V.
//
// r a power of two (k_lowrank_part_pow2): a thread loads eight 16-byte pieces of the chunk and,
// with each, the aligned 8-element block of x that holds the piece's rows (x is not staged). Its
// element i always falls in column (8 tid + i) mod r, so it keeps eight column sums; the threads
// sharing a set of columns are those equal modulo c = max(1, r / 8). Each wave adds them within
// rows of 16 lanes by DPP shifts of c, 2c, ... (the last c lanes of a row end with their class's
// sums), one LDS slot per row and class takes those, and after a single barrier thread k < r
// adds column k's 16 row slots in order.
template <int C>
__device__ __forceinline__ void class_row_sums(float* acc) {
  // acc[i] of lane L gains lanes L - C, L - 2C, ... of its row of 16 (same class modulo C)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if constexpr (C <= 1) acc[i] += dpp_f32<0x111, 0xF>(acc[i]);   // row_shr:1
    if constexpr (C <= 2) acc[i] += dpp_f32<0x112, 0xF>(acc[i]);   // row_shr:2
    if constexpr (C <= 4) acc[i] += dpp_f32<0x114, 0xF>(acc[i]);   // row_shr:4
    acc[i] += dpp_f32<0x118, 0xF>(acc[i]);                         // row_shr:8
  }
}

// element k (0..7) of 8 packed bf16, as fp32
__device__ __forceinline__ float bf16_element(const u32x4& b, int k) {
  const int d = k >> 1;
  const uint32_t w = d == 0 ? b.x : d == 1 ? b.y : d == 2 ? b.z : b.w;
  return __builtin_bit_cast(float, (k & 1) ? (w & 0xFFFF0000u) : (w << 16));
}

__global__ void k_lowrank_part_cols(const uint16_t* __restrict__ V, const uint16_t* __restrict__ x,
                                    float* __restrict__ part, int K, int r, int P);

template <int SH>
__global__ __launch_bounds__(kLrThreads) void k_lowrank_part_pow2(const uint16_t* __restrict__ V,
                                                                  const uint16_t* __restrict__ x,
                                                                  float* __restrict__ part, int K, int P) {
  constexpr int kRounds = kLrChunk / (kLrThreads * 8);
  constexpr int r = 1 << SH, sh = SH;
  __shared__ float slot[kLrThreads / 16][8][8];              // [row of 16 lanes][class][i]
  const int p = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  const int KC = kLrChunk >> sh, j0 = p * KC, rows = min(KC, K - j0);
  const int E = rows << sh;                                   // rows and E are multiples of 32
  const uint16_t* Vc = V + ((size_t)g * K + j0) * r;
  const u32x4* xc = reinterpret_cast<const u32x4*>(x + j0);   // j0 is a multiple of 256
  float* out = part + ((size_t)g * P + p) * r;
  u32x4 v[kRounds], xb[kRounds];
#pragma unroll
  for (int m = 0; m < kRounds; ++m) {
    const int e0 = (m * kLrThreads + tid) * 8;
    const bool in = e0 < E;
    v[m] = in ? *reinterpret_cast<const u32x4*>(Vc + e0) : u32x4{0u, 0u, 0u, 0u};
    // rows (e0 >> sh) .. of this piece; zeros past the chunk, as for v (0 * 0 adds nothing, where
    // a real x element could be infinite)
    xb[m] = in ? xc[(e0 >> sh) >> 3] : u32x4{0u, 0u, 0u, 0u};
  }
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
  for (int m = 0; m < kRounds; ++m) {
    const int e0 = (m * kLrThreads + tid) * 8;                // lanes past E hold zeros in v
    const int k0 = (e0 >> sh) & 7;
    const uint32_t w[4] = {v[m].x, v[m].y, v[m].z, v[m].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float vi = __builtin_bit_cast(float, (i & 1) ? (w[i >> 1] & 0xFFFF0000u) : (w[i >> 1] << 16));
      acc[i] = __builtin_fmaf(bf16_element(xb[m], k0 + (i >> sh)), vi, acc[i]);
    }
  }
  constexpr int c = r >= 8 ? r >> 3 : 1;
  class_row_sums<c>(acc);
  const int L = tid & 15;
  if (L >= 16 - c) {
#pragma unroll
    for (int i = 0; i < 8; ++i) slot[tid >> 4][L - (16 - c)][i] = acc[i];
  }
  __syncthreads();
  if (tid < r) {
    float t = 0.0f;
    if constexpr (r >= 8) {
      for (int row = 0; row < kLrThreads / 16; ++row) t += slot[row][tid >> 3][tid & 7];
    } else {
      for (int row = 0; row < kLrThreads / 16; ++row)
        for (int i = tid; i < 8; i += r) t += slot[row][0][i];
    }
    out[tid] = t;
  }
}

void launch_lowrank_part(const uint16_t* V, const uint16_t* x, float* ws, int K, int r, int P, int n_seg,
                         hipStream_t stream) {
  const dim3 grid((unsigned)P, (unsigned)n_seg);
  switch (r) {
    case 1: k_lowrank_part_pow2<0><<<grid, kLrThreads, 0, stream>>>(V, x, ws, K, P); break;
    case 2: k_lowrank_part_pow2<1><<<grid, kLrThreads, 0, stream>>>(V, x, ws, K, P); break;
    case 4: k_lowrank_part_pow2<2><<<grid, kLrThreads, 0, stream>>>(V, x, ws, K, P); break;
    case 8: k_lowrank_part_pow2<3><<<grid, kLrThreads, 0, stream>>>(V, x, ws, K, P); break;
    case 16: k_lowrank_part_pow2<4><<<grid, kLrThreads, 0, stream>>>(V, x, ws, K, P); break;
    case 32: k_lowrank_part_pow2<5><<<grid, kLrThreads, 0, stream>>>(V, x, ws, K, P); break;
    case 64: k_lowrank_part_pow2<6><<<grid, kLrThreads, 0, stream>>>(V, x, ws, K, P); break;
    default: k_lowrank_part_cols<<<grid, kLrThreads, 0, stream>>>(V, x, ws, K, r, P); break;
  }
}

// Other ranks (k_lowrank_part_cols): x staged in LDS, one column per thread, the workgroup's
// column slots added in order.
__global__ __launch_bounds__(kLrThreads) void k_lowrank_part_cols(const uint16_t* __restrict__ V,
                                                                  const uint16_t* __restrict__ x,
                                                                  float* __restrict__ part, int K, int r, int P) {
  __shared__ float l1[kLrThreads];
  __shared__ uint16_t xl[kLrChunk];
  const int p = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  const int KC = kLrChunk / r, j0 = p * KC, rows = min(KC, K - j0);
  const uint16_t* Vc = V + ((size_t)g * K + j0) * r;
  float* out = part + ((size_t)g * P + p) * r;
  for (int j = tid; j < rows; j += kLrThreads) xl[j] = x[j0 + j];
  __syncthreads();
  const int G = kLrThreads / r, q = tid / r, k = tid - q * r;
  float a = 0.0f;
  if (q < G)
    for (int j = q; j < rows; j += G) a = __builtin_fmaf(bf16_bits_to_f32(xl[j]), bf16_bits_to_f32(Vc[(size_t)j * r + k]), a);
  l1[tid] = a;
  __syncthreads();
  if (tid < r) {
    float t = 0.0f;
    for (int qq = 0; qq < G; ++qq) t += l1[qq * r + tid];
    out[tid] = t;
  }
}

SegTable seg_table(const attnq_nvfp4& W) {
  SegTable t;
  t.n_seg = W.n_seg;
  for (int i = 0; i < ATTNQ_MAX_SEGMENTS; ++i) t.end[i] = (i < W.n_seg) ? W.seg_end[i] : W.N;
  return t;
}

void launch_glu_loop(const attnq_nvfp4& W, const uint16_t* x, uint16_t* h, int act, hipStream_t stream) {
  const unsigned grid = (unsigned)((W.N / 2 + 3) / 4);
  k_gemv_nvfp4<2, 1, 1><<<grid, 256, 0, stream>>>(W.codes, W.scales, W.tensor_scale, seg_table(W), x, nullptr, W.N,
                                                  W.K, h, act);
}

template <int R, int KSPLIT>
void launch_nvfp4_loop(const attnq_nvfp4& W, const uint16_t* x, float* y, hipStream_t stream) {
  constexpr int rows_per_wg = R * (4 / KSPLIT);
  const unsigned grid = (unsigned)((W.N + rows_per_wg - 1) / rows_per_wg);
  k_gemv_nvfp4<R, KSPLIT><<<grid, 256, 0, stream>>>(W.codes, W.scales, W.tensor_scale, seg_table(W), x, y, W.N, W.K);
}

// The one-shot launchers refuse (launch nothing, return false) rows longer than the kernel's
// KSPLIT x S x 64 chunks, which is also the pitch of its x staging in LDS.
template <int R, int KSPLIT, int S, bool XL, int WAVES, bool XFIRST = false, int XI = 1>
bool launch_nvfp4_oneshot(const attnq_nvfp4& W, const uint16_t* x, float* y, hipStream_t stream) {
  if (W.K / 32 > KSPLIT * S * 64) return false;
  constexpr int rows_per_wg = R * (WAVES / KSPLIT);
  const unsigned grid = (unsigned)((W.N + rows_per_wg - 1) / rows_per_wg);
  k_gemv_nvfp4_oneshot<R, KSPLIT, S, XL, WAVES, XFIRST, XI><<<grid, 64 * WAVES, 0, stream>>>(
      W.codes, W.scales, W.tensor_scale, seg_table(W), x, y, W.N, W.K);
  return true;
}

int lowrank_parts(int K, int r) {
  const int KC = kLrChunk / r;
  return (K + KC - 1) / KC;
}

template <int R, int KSPLIT, int S, bool XL, int WAVES, bool XFIRST = false, int XI = 1>
bool launch_lr_oneshot(const attnq_nvfp4& W, const uint16_t* x, float* y, const LowRank& lr, hipStream_t stream) {
  if (W.K / 32 > KSPLIT * S * 64) return false;
  constexpr int rows_per_wg = R * (WAVES / KSPLIT);
  const unsigned grid = (unsigned)((W.N + rows_per_wg - 1) / rows_per_wg);
  k_gemv_nvfp4_oneshot<R, KSPLIT, S, XL, WAVES, XFIRST, XI, 2><<<grid, 64 * WAVES, 0, stream>>>(
      W.codes, W.scales, W.tensor_scale, seg_table(W), x, y, W.N, W.K, nullptr, 0, lr);
  return true;
}

template <int R, int KSPLIT>
void launch_lr_loop(const attnq_nvfp4& W, const uint16_t* x, float* y, const LowRank& lr, hipStream_t stream) {
  constexpr int rows_per_wg = R * (4 / KSPLIT);
  const unsigned grid = (unsigned)((W.N + rows_per_wg - 1) / rows_per_wg);
  k_gemv_nvfp4<R, KSPLIT, 2><<<grid, 256, 0, stream>>>(W.codes, W.scales, W.tensor_scale, seg_table(W), x, y, W.N, W.K,
                                                       nullptr, 0, lr);
}

// gate|up epilogue launches: one row pair per wave, 4 waves, F = N / 2 pairs, x loaded ahead of the
// weights (4 waves measured 3.104 -> 3.084 ms per token in the chained stream against 8)
template <int S>
bool launch_glu_oneshot(const attnq_nvfp4& W, const uint16_t* x, uint16_t* h, int act, hipStream_t stream) {
  if (W.K / 32 > S * 64) return false;
  const unsigned grid = (unsigned)((W.N / 2 + 3) / 4);
  k_gemv_nvfp4_oneshot<2, 1, S, true, 4, true, 3, 1><<<grid, 256, 0, stream>>>(
      W.codes, W.scales, W.tensor_scale, seg_table(W), x, nullptr, W.N, W.K, h, act);
  return true;
}

// Split-K shape: slices of at most 2 x 64 chunks (4096 elements) on 8 waves of two rows each, SK =
// ceil(chunks / 128) slices (4 <= SK <= 12), every slice non-empty; rows of fewer than 512 chunks
// (16384 elements) or more than 1536 (49152) are not split. For the down projection (672 chunks)
// that is 6 slices of 112 chunks, 2016 workgroups: in the token stream this measured 14.0 us against
// 14.2-14.9 us for 7 or 8 slices of two steps, 14.8 us for 4 slices of three steps, 15.6 us for 3
// of four, 14.5-15.0 us with four rows per wave, 15.3-17.0 us with one step per slice (11 or 12
// slices) and 17.0-17.4 us with one row per wave (16 waves).
constexpr int kSplitRows = 16;        // a tile: 8 waves x 2 rows
constexpr int kSplitS = 2, kSplitR = 2, kSplitWaves = kSplitRows / kSplitR;
int splitk_slices(int K) {
  const int cpr = K / 32;
  if (cpr < 512) return 0;
  const int sk = (cpr + kSplitS * 64 - 1) / (kSplitS * 64);
  if (sk < 2 || sk > kSplitMaxSlices) return 0;
  const int slice = (cpr + sk - 1) / sk;
  return (slice <= kSplitS * 64 && (sk - 1) * slice < cpr) ? sk : 0;
}

template <int SK, int EPI = 0>
void launch_splitk_sk(const attnq_nvfp4& W, const uint16_t* x, float* y, uint8_t* ws, hipStream_t stream,
                      const LowRank& lr = {}) {
  const unsigned tiles = (unsigned)((W.N + kSplitRows - 1) / kSplitRows);
  constexpr int kXI = (4 * kSplitS * 64 + 64 * kSplitWaves - 1) / (64 * kSplitWaves);   // x pieces per thread
  k_gemv_nvfp4_splitk<kSplitR, kSplitS, kSplitWaves, kXI, SK, EPI><<<tiles * SK, 64 * kSplitWaves, 0, stream>>>(
      W.codes, W.scales, W.tensor_scale, seg_table(W), x, y, W.N, W.K, ws, lr);
}

}  // namespace

// Launch table (timed per shape on MI355X, 31B-like shapes streamed cold, then A/B inside the
// token stream): rows of up to 6144 elements use the one-shot kernel with x loaded ahead of the
// weights (XFIRST: better inside the stream, where each layer's x is cold): the fused gate|up
// (43008 x 5376) with two rows per wave and 4 waves, q|k|v (6144 x 5376) with one row per wave and
// 4 waves, o (5376 x 4096, two steps) with one row per wave and 8 waves (after the branch-free
// staging, 8 waves for o and 4 for q|k|v measured 3.087 -> 3.077 ms per token against 4 and 8,
// and 4 waves for gate|up 3.102 -> 3.093 against 8; 16 waves, two rows per wave for q|k|v, one for
// gate|up and 2 waves for o were slower). Rows of at most 64 chunks (K <= 2048: the 1B-like and
// 1024 x 1152 shapes) take one step instead of two, which left 92 of every 128 lane loads of a
// 36-chunk row reloading a clamped chunk, with two rows per wave for tall weights; rows of 193 to
// 256 chunks (the 1B-like down, K = 6912) take four steps instead of the loop kernel. The 26-layer
// 1B-like stack measured 0.399 -> 0.329 ms per token, the 1024 x 1152 projection 2.62 -> 2.35 us.
// Long rows (the down projection, K = 21504) use the loop kernel with four rows per wave and
// K split over two waves (two row groups per workgroup): inside the token stream this beat
// splits of 1 and 4, 2 or 8 rows per wave, x staged in LDS, the one-shot kernel and a balanced
// walk with one workgroup per compute unit.
hipError_t launch_gemv_nvfp4(const attnq_nvfp4& W, const uint16_t* x, float* y, hipStream_t stream) {
  if (W.N == 0) return hipSuccess;
  const int cpr = W.K / 32;
  bool ok = true;
  if (W.K >= 16384)
    launch_nvfp4_loop<4, 2>(W, x, y, stream);
  else if (cpr <= 64 && W.N >= 8192)
    ok = launch_nvfp4_oneshot<2, 1, 1, true, 4, true, 1>(W, x, y, stream);    // K <= 2048, tall (1B-like gate|up 13824x1152): two rows per wave, one step
  else if (cpr <= 64)
    ok = launch_nvfp4_oneshot<1, 1, 1, true, 4, true, 1>(W, x, y, stream);    // K <= 2048: one row per wave, one step (x: 256 >= K/8)
  else if (cpr <= 128)
    ok = launch_nvfp4_oneshot<1, 1, 2, true, 8, true, 1>(W, x, y, stream);    // K <= 4096: one row per wave, two steps (x: 512 >= K/8)
  else if (cpr <= 192 && W.N >= 16384)
    ok = launch_nvfp4_oneshot<2, 1, 3, true, 4, true, 3>(W, x, y, stream);    // fused gate|up 43008x5376 (x: 3 x 256 >= K/8)
  else if (cpr <= 192)
    ok = launch_nvfp4_oneshot<1, 1, 3, true, 4, true, 3>(W, x, y, stream);    // fused q|k|v 6144x5376 (x: 3 x 256 >= K/8)
  else if (cpr <= 256)
    ok = launch_nvfp4_oneshot<1, 1, 4, true, 8, true, 2>(W, x, y, stream);    // K <= 8192 (1B-like down 1152x6912): four steps (x: 2 x 512 >= K/8)
  else
    launch_nvfp4_loop<2, 2>(W, x, y, stream);
  return ok ? hipGetLastError() : hipErrorInvalidValue;
}

// Workspace of the split-K GEMV: one record per row tile (0 for shapes that are not split).
int64_t gemv_nvfp4_splitk_workspace_bytes(int N, int K) {
  const int sk = splitk_slices(K);
  if (sk == 0 || N == 0) return 0;
  return (int64_t)((N + kSplitRows - 1) / kSplitRows) * kSplitRecordBytes;
}

hipError_t launch_gemv_nvfp4_splitk(const attnq_nvfp4& W, const uint16_t* x, float* y, void* ws, hipStream_t stream) {
  const int sk = splitk_slices(W.K);
  if (W.N == 0) return hipSuccess;
  if (sk == 0) return launch_gemv_nvfp4(W, x, y, stream);
  uint8_t* w = static_cast<uint8_t*>(ws);
  switch (sk) {
    case 4: launch_splitk_sk<4>(W, x, y, w, stream); break;
    case 5: launch_splitk_sk<5>(W, x, y, w, stream); break;
    case 6: launch_splitk_sk<6>(W, x, y, w, stream); break;
    case 7: launch_splitk_sk<7>(W, x, y, w, stream); break;
    case 8: launch_splitk_sk<8>(W, x, y, w, stream); break;
    case 9: launch_splitk_sk<9>(W, x, y, w, stream); break;
    case 10: launch_splitk_sk<10>(W, x, y, w, stream); break;
    case 11: launch_splitk_sk<11>(W, x, y, w, stream); break;
    case 12: launch_splitk_sk<12>(W, x, y, w, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// The allocation-free split-K entry point keeps its tile records in this device array: 1 MiB, 1260
// records, so weights of up to 20160 rows. Each GPU the library runs on holds its own copy until the
// process ends. Host code never names the array in a launch or a copy (its host-side name is not a
// device address): at a device's first call its address is taken once with hipGetSymbolAddress,
// with that device current, and kept per device; the array is cleared by a kernel then.
constexpr int64_t kScratchBytes = int64_t{1} << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
uint8_t* g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_of_current_device(hipStream_t stream, uint8_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    k_clear_words<<<256, 256, 0, stream>>>(static_cast<uint32_t*>(p), (int)(kScratchBytes / 4));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<uint8_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

int64_t gemv_nvfp4_splitk_noalloc_max_bytes() { return kScratchBytes; }

hipError_t launch_gemv_nvfp4_splitk_noalloc(const attnq_nvfp4& W, const uint16_t* x, float* y, hipStream_t stream) {
  if (gemv_nvfp4_splitk_workspace_bytes(W.N, W.K) == 0) return launch_gemv_nvfp4(W, x, y, stream);
  uint8_t* ws = nullptr;
  const hipError_t e = scratch_of_current_device(stream, &ws);
  if (e != hipSuccess) return e;
  return launch_gemv_nvfp4_splitk(W, x, y, ws, stream);
}

// Small-M on the batch-1 walk: M = 1 .. 4 tokens and rows of at most 192 chunks (o-like rows of up
// to 128 chunks: one row per wave, two steps, 8 waves; tall weights: two rows per wave; otherwise
// one row per wave, 8 waves). The x staging of up to 4 tokens (34 KB for o-like rows) holds a
// compute unit to 4 workgroups, so o-like rows take 8 waves per workgroup, not 4: at M = 4 the
// 31B-like o measured 7.6 -> 6.4 us per launch. Returns false (nothing launched) for other shapes.
template <int MT>
void launch_tokens_mt(const attnq_nvfp4& W, const uint16_t* X, int ldx, float* Y, int ldy, hipStream_t stream) {
  const int cpr = W.K / 32;
  const SegTable t = seg_table(W);
  if (cpr <= 128)          // x: 512 pieces >= K / 8
    k_gemm_nvfp4_tokens<MT, 1, 2, 8, 1><<<(W.N + 7) / 8, 512, 0, stream>>>(W.codes, W.scales, W.tensor_scale, t, X,
                                                                           ldx, Y, ldy, W.N, W.K);
  else if (W.N >= 16384)   // x: 2 x 512 pieces >= K / 8
    k_gemm_nvfp4_tokens<MT, 2, 3, 8, 2><<<(W.N + 15) / 16, 512, 0, stream>>>(W.codes, W.scales, W.tensor_scale, t,
                                                                             X, ldx, Y, ldy, W.N, W.K);
  else
    k_gemm_nvfp4_tokens<MT, 1, 3, 8, 2><<<(W.N + 7) / 8, 512, 0, stream>>>(W.codes, W.scales, W.tensor_scale, t, X,
                                                                           ldx, Y, ldy, W.N, W.K);
}

// Runtime low-rank product over a shared NVFP4 block: the partial sums of t = V^T x (one
// workgroup per 16 KB chunk of V and segment), then the streaming GEMV with the s / U t epilogue,
// in the plain GEMV's launch configurations for gate|up (4 waves: the low-rank stream 4.290 ->
// 4.248 ms against 8), rows of 193 to 256 chunks and the long rows; q|k|v and o keep 8 and 4 waves
// (the plain GEMV's 4 and 8 measured the same in the low-rank stream), and rows of up to 64 chunks
// two steps, the second masked. Each row is summed in the plain GEMV's order, so with r = 0 and no
// s the result equals attnq_gemv_nvfp4's bit for bit.
int64_t lowrank_workspace_floats(int K, int n_seg, int r) {
  return r == 0 ? 0 : (int64_t)n_seg * lowrank_parts(K, r) * r;
}

hipError_t launch_gemv_nvfp4_lowrank(const attnq_nvfp4& W, const uint16_t* s, const uint16_t* U, const uint16_t* V,
                                     int r, const uint16_t* x, float* ws, float* y, hipStream_t stream) {
  if (W.N == 0) return hipSuccess;
  LowRank lr{s, U, ws, r, 0};
  if (r > 0) {
    lr.P = lowrank_parts(W.K, r);
    launch_lowrank_part(V, x, ws, W.K, r, lr.P, W.n_seg, stream);
  }
  const int cpr = W.K / 32;
  bool ok = true;
  if (W.K >= 16384)
    launch_lr_loop<4, 2>(W, x, y, lr, stream);
  else if (cpr <= 128)
    ok = launch_lr_oneshot<1, 1, 2, true, 4, true, 2>(W, x, y, lr, stream);
  else if (cpr <= 192 && W.N >= 16384)
    ok = launch_lr_oneshot<2, 1, 3, true, 4, true, 3>(W, x, y, lr, stream);
  else if (cpr <= 192)
    ok = launch_lr_oneshot<1, 1, 3, true, 8, true, 2>(W, x, y, lr, stream);
  else if (cpr <= 256)
    ok = launch_lr_oneshot<1, 1, 4, true, 8, true, 2>(W, x, y, lr, stream);
  else
    launch_lr_loop<2, 2>(W, x, y, lr, stream);
  return ok ? hipGetLastError() : hipErrorInvalidValue;
}

// The low-rank product with the split-K GEMV: rows split into at most 6 K slices (16384 to 24576
// elements: the 31B-like down projection), whose records hold the row-term shares next to the
// partial sums; other shapes run launch_gemv_nvfp4_lowrank. The row terms are summed in another
// order than there (slices of i instead of the wave's K split), so the two agree within fp32
// rounding, not bit for bit.
hipError_t launch_gemv_nvfp4_lowrank_splitk(const attnq_nvfp4& W, const uint16_t* s, const uint16_t* U,
                                            const uint16_t* V, int r, const uint16_t* x, float* ws, void* split_ws,
                                            float* y, hipStream_t stream) {
  if (W.N == 0) return hipSuccess;
  const int sk = splitk_slices(W.K);
  if (sk == 0 || 2 * sk > kSplitMaxSlices) return launch_gemv_nvfp4_lowrank(W, s, U, V, r, x, ws, y, stream);
  LowRank lr{s, U, ws, r, 0};
  if (r > 0) {
    lr.P = lowrank_parts(W.K, r);
    launch_lowrank_part(V, x, ws, W.K, r, lr.P, W.n_seg, stream);
  }
  uint8_t* w = static_cast<uint8_t*>(split_ws);
  switch (sk) {
    case 4: launch_splitk_sk<4, 2>(W, x, y, w, stream, lr); break;
    case 5: launch_splitk_sk<5, 2>(W, x, y, w, stream, lr); break;
    case 6: launch_splitk_sk<6, 2>(W, x, y, w, stream, lr); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// gate|up with its activation: the one-shot kernel stages x in LDS for rows of up to 6144
// elements (the fused gate|up shapes); longer rows walk K in the loop kernel.
hipError_t launch_gemv_nvfp4_glu(const attnq_nvfp4& W, const uint16_t* x, int act, uint16_t* h, hipStream_t stream) {
  if (W.N == 0) return hipSuccess;
  const int cpr = W.K / 32;
  bool ok = true;
  if (cpr <= 64)
    ok = launch_glu_oneshot<1>(W, x, h, act, stream);
  else if (cpr <= 128)
    ok = launch_glu_oneshot<2>(W, x, h, act, stream);
  else if (cpr <= 192)
    ok = launch_glu_oneshot<3>(W, x, h, act, stream);
  else
    launch_glu_loop(W, x, h, act, stream);
  return ok ? hipGetLastError() : hipErrorInvalidValue;
}

bool launch_gemm_nvfp4_tokens(const attnq_nvfp4& W, const uint16_t* X, int M, int ldx, float* Y, int ldy,
                              hipStream_t stream) {
  if (W.K / 32 > 192 || M < 1 || M > 4) return false;
  if (M == 1) launch_tokens_mt<1>(W, X, ldx, Y, ldy, stream);
  else if (M == 2) launch_tokens_mt<2>(W, X, ldx, Y, ldy, stream);
  else if (M == 3) launch_tokens_mt<3>(W, X, ldx, Y, ldy, stream);
  else launch_tokens_mt<4>(W, X, ldx, Y, ldy, stream);
  return true;
}

hipError_t launch_gemv_bf16(const uint16_t* W, int N, int K, const uint16_t* x, float* y, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  // rows of up to 4096 / 5632 elements: one row per wave, every load issued at once (8 / 11 steps),
  // eight waves per workgroup (measured ahead of 2, 4 and 16 on the lm_head and q|k|v shapes);
  // longer rows walk K two rows per wave, four chunks in flight
  const int cpr = K / 8;
  if (cpr <= 512) {
    k_gemv_bf16_oneshot<1, 8, 8><<<(N + 7) / 8, 512, 0, stream>>>(W, x, y, N, K);
    return hipGetLastError();
  }
  if (cpr <= 704) {
    k_gemv_bf16_oneshot<1, 11, 8><<<(N + 7) / 8, 512, 0, stream>>>(W, x, y, N, K);
    return hipGetLastError();
  }
  constexpr int R = 2;
  const unsigned grid = (unsigned)((N + 4 * R - 1) / (4 * R));
  k_gemv_bf16<R><<<grid, 256, 0, stream>>>(W, x, y, N, K);
  return hipGetLastError();
}

}  // namespace attnq
