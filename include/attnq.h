/*
 * attnq.h -- C ABI of libattnq.so: load-time NVFP4 weight-only RTN quantization and the
 * batch-1 / tiny-batch decode projections y = x * W_eff^T on AMD Instinct MI355X (gfx950).
 *
 * Source of the operations (documentation pages of the AttnQuant / weightless projects):
 *   - theta bundle and reconstruction W_eff = s*W0 + U*V^T: AttnQuant landing page,
 *     "How it works"; weightless "GPU and cache acceleration", "Architecture decisions /
 *     Precompute-outside (the fast path)".
 *   - NVFP4 round-to-nearest quantization at load, packed uint8 codes plus float8 block
 *     scales: "GPU acceleration", "NVFP4 quantization"; landing page, "Results";
 *     "Throughput", "What quantization actually saves" (an E4M3 scale byte for each block
 *     of 16 elements, 0.5625 B per element).
 *   - the decode GEMVs that consume fp4 directly with no dequant pass, fused Q/K/V, the bf16
 *     tied lm_head: "GPU acceleration", "Where GPU time goes" and "Q/K/V fusion";
 *     "Throughput", "The NVFP4 MLP kernels are the least bandwidth-efficient on the step".
 *   - small-M products for speculative verification (gamma = 3 drafts plus one) and batch 8:
 *     "Throughput", "Speculative decoding".
 *
 * Conventions shared by every call:
 *   - Memory: every array argument is DEVICE memory owned by the caller; descriptor structs
 *     are HOST memory read during the call only. The library allocates nothing and, apart from
 *     the scratch array of attnq_gemv_nvfp4_splitk_noalloc, keeps no mutable global state, so
 *     calls from several host threads are safe.
 *   - Asynchrony: each call validates its arguments on the host, enqueues its kernels on
 *     `stream` (a hipStream_t; NULL is the default stream) and returns. It never
 *     synchronizes, copies to or from the host, or reads device data on the host.
 *   - Errors: argument errors are returned synchronously before anything is enqueued; a
 *     failed launch returns ATTNQ_ERR_HIP. Bad data is reported in-band: a projection whose
 *     weights hold a NaN or an infinity gets tensor scale NaN, so its outputs are NaN.
 *   - bf16 values travel as uint16_t bit patterns; outputs y / Y are fp32.
 *   - Shapes: K must be a positive multiple of 32 (two scale blocks per 16-byte code chunk);
 *     N == 0 (or M == 0) is a valid no-op, and a pointer to such an empty array may be NULL.
 */
#ifndef ATTNQ_H
#define ATTNQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Exported entry points (the library is built with hidden default visibility). */
#define ATTNQ_API __attribute__((visibility("default")))

typedef enum attnq_status {
  ATTNQ_OK = 0,
  ATTNQ_ERR_NULL = 1,    /* a required pointer is NULL */
  ATTNQ_ERR_SHAPE = 2,   /* a size is out of range (see each call) */
  ATTNQ_ERR_ALIGN = 3,   /* a device pointer is not aligned as documented */
  ATTNQ_ERR_SEGMENT = 4, /* segment table or segment index inconsistent */
  ATTNQ_ERR_LAYOUT = 5,  /* unknown packed-weight layout id */
  ATTNQ_ERR_HIP = 6      /* a kernel launch failed */
} attnq_status;

/* hipStream_t, passed opaquely so that this header needs no HIP include. */
typedef void* attnq_stream;

/* One projection's theta bundle (landing page, "How it works").
 *   W0 [N][K] bf16 row-major, 16-byte aligned. Several bundles may point at one W0
 *      (a shared block).
 *   s  [N] bf16 per-row scale, or NULL for s = 1.
 *   U  [N][r] bf16, V [K][r] bf16 (row-major), both NULL iff r == 0; 0 <= r <= 64.
 * A plain bf16 weight W is the bundle {W, NULL, NULL, NULL, N, K, 0}. */
typedef struct attnq_theta {
  const uint16_t* W0;
  const uint16_t* s;
  const uint16_t* U;
  const uint16_t* V;
  int32_t N;
  int32_t K;
  int32_t r;
} attnq_theta;

#define ATTNQ_MAX_SEGMENTS 4
#define ATTNQ_MAX_BATCH 8   /* theta bundles per attnq_quantize_nvfp4_staged_batch call */
#define ATTNQ_LAYOUT_ROW_MAJOR 0

/* An NVFP4 weight [N][K], possibly several projections fused along N ("Q/K/V fusion":
 * q, k, v rows concatenated; gate and up likewise). Segment i covers rows
 * [seg_end[i-1], seg_end[i]) (seg_end[-1] = 0) and has its own tensor scale.
 *   codes  [N][K/2] u8, 16-byte aligned: element 2j of a row in the low nibble of byte j,
 *          element 2j+1 in the high nibble; a nibble is sign<<3 | E2M1 magnitude index
 *          (0, 0.5, 1, 1.5, 2, 3, 4, 6).
 *   scales [N][K/16] E4M3FN, 4-byte aligned: block b scales elements [16b, 16b+16) of a row.
 *   tensor_scale [n_seg] fp32, 4-byte aligned: the dequantization multiplier of a segment.
 *   weight[n][k] = e2m1(code) * e4m3(scale[n][k/16]) * tensor_scale[segment of n].
 *   1 <= n_seg <= 4, seg_end strictly ascending, seg_end[n_seg-1] == N.
 *   N * K/2 <= 2^32: the kernels address codes and scales with 32-bit byte offsets (every call
 *   that takes an attnq_nvfp4 returns ATTNQ_ERR_SHAPE beyond that).
 *   layout: ATTNQ_LAYOUT_ROW_MAJOR (0) is the only layout. */
typedef struct attnq_nvfp4 {
  uint8_t* codes;
  uint8_t* scales;
  float* tensor_scale;
  int32_t N;
  int32_t K;
  int32_t n_seg;
  int32_t seg_end[ATTNQ_MAX_SEGMENTS];
  int32_t layout;
} attnq_nvfp4;

/* W_eff = s*W0 + U*V^T (landing page "How it works"; weightless "Precompute-outside").
 * Rounding: acc = 0, acc += U[i][k]*V[j][k] in fp32 for k ascending, w = s_i*W0[i][j] + acc
 * (skipped add when r == 0), one fp32 rounding per step, then bf16 round-to-nearest-even.
 * With s = NULL and r = 0 the output equals W0 bit for bit.
 * W_eff [N][K] bf16, 16-byte aligned, must not overlap the inputs.
 * Errors: NULL theta/W0/W_eff or (r > 0 and NULL U/V); N < 0, K not a positive multiple of
 * 32, r outside [0, 64]; misaligned W0 / W_eff. */
ATTNQ_API attnq_status attnq_reconstruct(const attnq_theta* theta, uint16_t* W_eff, attnq_stream stream);

/* Reconstruct (as attnq_reconstruct, in registers) and round-to-nearest quantize one
 * projection into segment `seg` of `dst` ("NVFP4 quantization"; landing page "Results").
 * Per segment: amax = max |W_eff|; ts = fl32(amax / 2688) (2688 = 6 * 448);
 * per 16-element block: S = E4M3(fl32(bamax / fl32(6*ts))) rounded to nearest, ties to even,
 * saturating at 448; d = fl32(e4m3(S)*ts); each element: q = fl32(w / d) rounded to the E2M1
 * grid, ties to the even code, saturating at 6, sign of w kept; S == 0 gives magnitude 0.
 * amax == 0 gives ts = 0 and all scales 0. A NaN/inf in the segment gives ts = NaN, every
 * scale 0x7F and every code byte 0.
 * theta->N must equal the segment's row count and theta->K == dst->K. The segment's
 * tensor_scale slot is zeroed and then accumulates the tensor scale while the call runs (three
 * kernels in stream order); other segments of dst are untouched.
 * Errors: as attnq_reconstruct, plus ATTNQ_ERR_SEGMENT for a bad seg or row count and
 * ATTNQ_ERR_LAYOUT for an unknown layout. */
ATTNQ_API attnq_status attnq_quantize_nvfp4(const attnq_theta* theta, const attnq_nvfp4* dst, int32_t seg,
                                  attnq_stream stream);

/* The same result as attnq_quantize_nvfp4, bit for bit, with W_eff rebuilt once instead of twice
 * ("Throughput", "What quantization actually saves": the rebuild is load-time work). The first
 * kernel rebuilds W_eff, folds its amax into the tensor scale and writes it as bf16 into the
 * workspace; the second rounds it to NVFP4 from there. At r == 0 there is nothing to rebuild and
 * the call is attnq_quantize_nvfp4 (the workspace is not touched and may be NULL).
 * workspace: caller-owned device memory of at least attnq_quantize_nvfp4_staged_workspace(N, K, r)
 * bytes (2 N K for r > 0), 256-byte aligned, overlapping neither theta's arrays nor dst; its
 * contents on entry do not matter and it holds W_eff on return. Calls that share a workspace must
 * be ordered (one stream).
 * Errors: as attnq_quantize_nvfp4, plus ATTNQ_ERR_NULL for a NULL workspace, ATTNQ_ERR_SHAPE for
 * workspace_bytes below the size, ATTNQ_ERR_ALIGN for a misaligned workspace (r > 0 only). */
ATTNQ_API attnq_status attnq_quantize_nvfp4_staged(const attnq_theta* theta, const attnq_nvfp4* dst, int32_t seg,
                                                   void* workspace, int64_t workspace_bytes, attnq_stream stream);

/* Workspace bytes for attnq_quantize_nvfp4_staged on an [N][K] projection of rank r: 2 N K for
 * r > 0 and N, K > 0, else 0. */
ATTNQ_API int64_t attnq_quantize_nvfp4_staged_workspace(int32_t N, int32_t K, int32_t r);

/* attnq_quantize_nvfp4_staged for `count` (0..ATTNQ_MAX_BATCH) theta bundles at once, e.g. the
 * projections of one layer at load time ("Throughput", "What quantization actually saves"): bundle i
 * is quantized into segment segs[i] of dsts[i], each with the single call's result bit for bit.
 * The work takes three kernels in stream order instead of three per bundle: the tensor-scale slots
 * are zeroed together, the rank-16 bundles of whole 32 x 128 tiles are rebuilt in one grid (their
 * tiles cut into equal runs, one per wave), other bundles' amax passes follow one by one, and one
 * grid quantizes every bundle.
 * thetas, dsts, segs: host arrays of `count` entries, each validated as attnq_quantize_nvfp4_staged
 * validates its arguments; no two entries may name the same segment of the same weight.
 * workspace: caller-owned device memory of at least
 * attnq_quantize_nvfp4_staged_batch_workspace(thetas, count) bytes (bundle i's W_eff at the sum of
 * the earlier bundles' 2 N K, each rounded up to 256 bytes), 256-byte aligned, overlapping no
 * input or output; contents on entry do not matter. NULL is allowed when that size is 0.
 * Errors: as attnq_quantize_nvfp4_staged for any entry; ATTNQ_ERR_NULL for NULL arrays with
 * count > 0; ATTNQ_ERR_SHAPE for count outside [0, ATTNQ_MAX_BATCH]; ATTNQ_ERR_SEGMENT for a
 * segment named twice. Nothing is launched when an error is returned. */
ATTNQ_API attnq_status attnq_quantize_nvfp4_staged_batch(const attnq_theta* thetas, const attnq_nvfp4* dsts,
                                                         const int32_t* segs, int32_t count, void* workspace,
                                                         int64_t workspace_bytes, attnq_stream stream);

/* Workspace bytes for attnq_quantize_nvfp4_staged_batch: the sum over the bundles of
 * attnq_quantize_nvfp4_staged_workspace(N, K, r), each rounded up to a multiple of 256; -1 for
 * count outside [0, ATTNQ_MAX_BATCH] or a NULL array with count > 0. */
ATTNQ_API int64_t attnq_quantize_nvfp4_staged_batch_workspace(const attnq_theta* thetas, int32_t count);

/* y[n] = sum_k x[k] * weight[n][k] for an NVFP4 weight: one kernel that reads codes and
 * scales once and decodes fp4 in registers ("Where GPU time goes": no dequant pass).
 * x [K] bf16 16-byte aligned; y [N] fp32 4-byte aligned, must not overlap x or the weight.
 * Accumulation is fp32. Errors (checked on the host, nothing launched): ATTNQ_ERR_NULL for a NULL
 * weight, tensor_scale or x, or NULL codes / scales / y with N > 0; ATTNQ_ERR_LAYOUT for an
 * unknown layout; ATTNQ_ERR_SHAPE for N < 0, K not a positive multiple of 32 or N * K/2 > 2^32;
 * ATTNQ_ERR_SEGMENT for a segment table that is not strictly increasing up to N;
 * ATTNQ_ERR_ALIGN for a misaligned pointer; ATTNQ_ERR_HIP if the launch fails. */
ATTNQ_API attnq_status attnq_gemv_nvfp4(const attnq_nvfp4* W, const uint16_t* x, float* y,
                              attnq_stream stream);

/* The same product y[n] = sum_k x[k] * weight[n][k] with K split across workgroups for long rows
 * ("Throughput", "The NVFP4 MLP kernels are the least bandwidth-efficient on the step": the down
 * projection's launch filled too few compute units, and splitting K was the remedy named there).
 * For rows of 16384 to 49152 elements (K = 21504 for the 31B-like down projection) one kernel runs
 * the rows in tiles of 16, each tile's K in SK = ceil(K / 4096) slices (4 <= SK <= 12) on separate
 * workgroups; each workgroup writes its raw partial sums to the workspace, and the workgroup that
 * arrives last at the tile's ticket adds the SK partials of each row in slice order, applies the
 * tensor scale and stores y (no workgroup waits on another). The slices are added in a fixed
 * order, so repeated calls give identical bits. Shorter rows (or rows of more than 49152
 * elements) run exactly as attnq_gemv_nvfp4 and leave the workspace untouched.
 * ws: caller-owned device memory of at least attnq_gemv_nvfp4_splitk_workspace(N, K) bytes,
 * 256-byte aligned. It holds one 832-byte record per tile of 16 rows, at a stride that does not
 * depend on the weight: a ticket (the first 4 bytes of the record) and the tile's partial sums.
 * Fill the whole workspace with zeros once after allocating it; every call leaves the tickets
 * zero again, so one workspace serves any number of calls and any weights whose size query does
 * not exceed it. Calls that share one workspace must be ordered on one stream.
 * Errors: as attnq_gemv_nvfp4; ATTNQ_ERR_NULL for a NULL ws that is needed; ATTNQ_ERR_SHAPE for
 * ws_bytes below the size the shape needs; ATTNQ_ERR_ALIGN for a misaligned ws. */
ATTNQ_API attnq_status attnq_gemv_nvfp4_splitk(const attnq_nvfp4* W, const uint16_t* x, float* y, void* ws,
                                     int64_t ws_bytes, attnq_stream stream);

/* attnq_gemv_nvfp4_splitk without a workspace argument and without any allocation, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). The tile records live in a 1 MiB array inside the library, one per GPU,
 * held until the process ends; the first call on a device looks up that device's copy and clears
 * it with a kernel on `stream`. Shapes that need more than 1 MiB of records (more than 20160 rows,
 * for split rows) return ATTNQ_ERR_SHAPE; shapes that are not split run as attnq_gemv_nvfp4. The
 * results equal attnq_gemv_nvfp4_splitk's bit for bit. Every call on one GPU shares that GPU's
 * array (each call leaves its tickets zero), so calls that overlap on one GPU -- on different
 * streams, or from several host threads without stream ordering -- race and must not be made.
 * `stream` must belong to the current device. Errors: as attnq_gemv_nvfp4_splitk. */
ATTNQ_API attnq_status attnq_gemv_nvfp4_splitk_noalloc(const attnq_nvfp4* W, const uint16_t* x, float* y,
                                             attnq_stream stream);

/* Bytes of workspace attnq_gemv_nvfp4_splitk needs for an [N][K] weight (0 when that shape is not
 * split), or -1 if N < 0 or K is not a positive multiple of 32. Host only, no GPU call. */
ATTNQ_API int64_t attnq_gemv_nvfp4_splitk_workspace(int32_t N, int32_t K);

/* Activations of the gate|up epilogue (attnq_gemv_nvfp4_glu). The pages do not name the model's
 * activation, so it is a parameter:
 *   GELU_TANH: 0.5 g (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3)))
 *   SILU:      g / (1 + exp(-g))
 *   IDENTITY:  g (the plain product gate * up) */
#define ATTNQ_ACT_GELU_TANH 0
#define ATTNQ_ACT_SILU 1
#define ATTNQ_ACT_IDENTITY 2

/* Fused gate|up projection with its activation, the input of the down projection
 * (weightless "GPU and cache acceleration", "Future work": gate/up fusion on the pattern of the
 * Q/K/V fusion). W holds two segments of F = N/2 rows each, gate rows then up rows
 * (seg_end = {F, N}). For j < F:
 *   g_j = sum_k x[k] * weight[j][k],  u_j = sum_k x[k] * weight[F + j][k]   (fp32, as in
 *         attnq_gemv_nvfp4; for rows of up to 6144 elements they equal its y[j] and y[F + j]
 *         bit for bit, longer rows add their partial sums in another order),
 *   h[j] = bf16_rne(fl32(act(g_j) * u_j)), the activation evaluated in fp32.
 * One kernel, no fp32 y round trip. x [K] bf16 16-byte aligned; h [F] bf16 2-byte aligned, must
 * not overlap x or the weight.
 * Errors: as attnq_gemv_nvfp4; ATTNQ_ERR_SEGMENT unless n_seg == 2 and seg_end[0] * 2 == N;
 * ATTNQ_ERR_SHAPE for an unknown act. */
ATTNQ_API attnq_status attnq_gemv_nvfp4_glu(const attnq_nvfp4* W, const uint16_t* x, int32_t act, uint16_t* h,
                                  attnq_stream stream);

/* Runtime low-rank product over a shared NVFP4 block, the weight never rebuilt: for a row n of
 * segment g (each segment is one projection with its own factors, as in a fused q|k|v),
 *   y[n] = s[n] * (sum_k x[k] * weight0[n][k]) + sum_j U[n][j] * t[g][j],  t[g][j] = sum_k x[k] * V[g][k][j]
 * ("Throughput", "The runtime reconstruction path does not reach dense parity": W0 and the
 * low-rank delta applied on every forward pass; weightless "GPU and cache acceleration",
 * "Architecture decisions / Custom-op kernel": the W0 dot product and the low-rank delta fused in
 * one kernel with nothing materialized; "Future work / Trained weight sharing": a shared NVFP4 W0
 * plus a bf16 low-rank pair). W0 is an NVFP4 weight [N][K] that several projections may share
 * (each call reads it once); s [N] bf16 or NULL (s = 1); U [N][r] and V [n_seg][K][r] bf16
 * row-major, NULL when r == 0 (U may also be NULL when N == 0), 0 <= r <= 64.
 * ws is a caller-owned fp32 workspace of at least attnq_gemv_nvfp4_lowrank_workspace(K, n_seg, r)
 * values (NULL when r == 0); it receives partial sums of V[g]^T x, P per segment, each over
 * floor(16384 / r) consecutive k: ws[(g * P + p) * r + j], P = ceil(K / floor(16384 / r)).
 * Two kernels in stream order: the partial sums, then the streaming GEMV, which reduces them to
 * t and applies s and U t in its epilogue. fp32 arithmetic; every sum is taken in a fixed order,
 * so repeated calls give identical bits. x and V 16-byte aligned, y and ws 4-byte aligned, s and
 * U 2-byte aligned; y and ws must not overlap the inputs or each other. Calls that share one ws
 * must be ordered on one stream. Errors: as attnq_gemv_nvfp4; r outside [0, 64] is
 * ATTNQ_ERR_SHAPE. */
ATTNQ_API attnq_status attnq_gemv_nvfp4_lowrank(const attnq_nvfp4* W0, const uint16_t* s, const uint16_t* U,
                                      const uint16_t* V, int32_t r, const uint16_t* x, float* ws, float* y,
                                      attnq_stream stream);

/* The runtime low-rank product of attnq_gemv_nvfp4_lowrank (the same per-row definition: "AttnQuant
 * inference for MAX", "How it works"; the GEMV epilogue as in "GPU and cache acceleration", "Future
 * work") on the split-K GEMV of attnq_gemv_nvfp4_splitk, for rows of 16384 to 24576 elements (the
 * down projection's K = 21504, which the plain low-rank call reads with one workgroup per row group):
 * each K slice adds its share of the row terms sum_i U[n][i mod r] * t_i next to its partial sums,
 * and the workgroup that arrives last at a tile's ticket adds both in slice order and stores
 * y = (partial sums) * ts * s + (row terms). Other shapes run attnq_gemv_nvfp4_lowrank, and
 * split_ws is then not touched. ws: as for attnq_gemv_nvfp4_lowrank. split_ws: caller-owned
 * device memory of at least attnq_gemv_nvfp4_splitk_workspace(N, K) bytes, 256-byte aligned,
 * filled with zeros once after allocating it (every call leaves its tickets zero; it may be shared
 * with attnq_gemv_nvfp4_splitk calls ordered on one stream). The row terms are summed in another
 * order than in attnq_gemv_nvfp4_lowrank, so the two agree within fp32 rounding; repeated calls
 * give identical bits. Errors: as attnq_gemv_nvfp4_lowrank, and for split_ws as
 * attnq_gemv_nvfp4_splitk's ws (ATTNQ_ERR_NULL, ATTNQ_ERR_SHAPE when split_ws_bytes is too small,
 * ATTNQ_ERR_ALIGN). */
ATTNQ_API attnq_status attnq_gemv_nvfp4_lowrank_splitk(const attnq_nvfp4* W0, const uint16_t* s, const uint16_t* U,
                                                       const uint16_t* V, int32_t r, const uint16_t* x, float* ws,
                                                       void* split_ws, int64_t split_ws_bytes, float* y,
                                                       attnq_stream stream);

/* Number of fp32 values the workspace of attnq_gemv_nvfp4_lowrank needs for a weight of row length
 * K with n_seg segments at rank r (0 when r == 0), or -1 if K, n_seg or r is out of range. Host
 * only, no GPU call. */
ATTNQ_API int64_t attnq_gemv_nvfp4_lowrank_workspace(int32_t K, int32_t n_seg, int32_t r);

/* y[n] = sum_k x[k] * W[n][k] for a bf16 weight [N][K], row-major: the tied lm_head, which the
 * pages keep in bf16, and projections left in bf16 ("Where GPU time goes": the bf16 GEMV
 * families next to the NVFP4 ones). W and x 16-byte aligned, y 4-byte aligned and not
 * overlapping W or x; fp32 accumulation. Errors: ATTNQ_ERR_SHAPE for N < 0 or K not a positive
 * multiple of 32; ATTNQ_ERR_NULL for a NULL x, or a NULL W / y with N > 0; ATTNQ_ERR_ALIGN;
 * ATTNQ_ERR_HIP if the launch fails. */
ATTNQ_API attnq_status attnq_gemv_bf16(const uint16_t* W, int32_t N, int32_t K, const uint16_t* x, float* y,
                             attnq_stream stream);

/* Y[m][n] = sum_k X[m][k] * weight[n][k] for 0 <= M <= 16 token rows (speculative verify at
 * gamma + 1 = 4, batch 8). X row m at X + m*ldx (bf16, ldx >= K, ldx % 8 == 0, X 16-byte
 * aligned, (M - 1)*ldx + K < 2^30); Y row m at Y + m*ldy (fp32, ldy >= N, Y 4-byte aligned).
 * M <= 4 with rows of at most 6144 elements runs the batch-1 GEMV walk (each row of Y then equals
 * attnq_gemv_nvfp4 of that token bit for bit); other shapes use the MFMA matrix cores. fp32
 * accumulation. Errors: as attnq_gemv_nvfp4; M outside [0, 16] or a stride or extent out of
 * range is ATTNQ_ERR_SHAPE. */
ATTNQ_API attnq_status attnq_gemm_nvfp4_small_m(const attnq_nvfp4* W, const uint16_t* X, int32_t M,
                                      int32_t ldx, float* Y, int32_t ldy, attnq_stream stream);

/* The small-M product of attnq_gemm_nvfp4_small_m with K cut into slices on separate workgroups
 * ("Throughput", "Speculative decoding": the verify pass at gamma + 1 = 4 tokens; batch 8): for
 * rows of more than 6144 elements, and for weights of at least 16384 rows at M > 4 (the down and
 * fused gate|up projections), one kernel reads each slice's weights the
 * way the batch-1 GEMV does (all of a slice's loads issued at once), turns them into matrix-core
 * operands through LDS and writes the slice's raw partial sums to the workspace; a second kernel,
 * in stream order, adds the slices in slice order, applies the tensor scale and stores Y. Repeated
 * calls give identical bits. A shape whose K fits one slice (1024 elements) stores Y from the first
 * kernel and needs no workspace. Other shapes run exactly as attnq_gemm_nvfp4_small_m.
 * ws: caller-owned device memory of at least attnq_gemm_nvfp4_small_m_splitk_workspace(N, K, M)
 * bytes (0: not needed, ws may be NULL), 256-byte aligned, contents irrelevant on entry and
 * overwritten; calls that share one workspace must be ordered on one stream.
 * Errors: as attnq_gemm_nvfp4_small_m; ATTNQ_ERR_NULL for a NULL ws that is needed,
 * ATTNQ_ERR_SHAPE for ws_bytes below the size the shape needs, ATTNQ_ERR_ALIGN for a misaligned ws. */
ATTNQ_API attnq_status attnq_gemm_nvfp4_small_m_splitk(const attnq_nvfp4* W, const uint16_t* X, int32_t M,
                                             int32_t ldx, float* Y, int32_t ldy, void* ws, int64_t ws_bytes,
                                             attnq_stream stream);

/* Bytes of workspace attnq_gemm_nvfp4_small_m_splitk needs for an [N][K] weight and M tokens (0 when
 * that shape has no slices), or -1 if N < 0, K is not a positive multiple of 32 or M is outside
 * [0, 16]. Host only, no GPU call. */
ATTNQ_API int64_t attnq_gemm_nvfp4_small_m_splitk_workspace(int32_t N, int32_t K, int32_t M);

/* Measurement aid, not part of the decode path: read a_bytes at a and then b_bytes at b once, as a
 * plain streaming read (16-byte non-temporal loads, four in flight per lane, 4096 workgroups of 256
 * threads: a grid-stride walk, or one contiguous stretch per workgroup from 1 GiB up) that writes
 * nothing in practice. Its duration over a weight's
 * codes and scales is the practical read ceiling of that weight's GEMV ("Throughput", "What a
 * decode step is actually made of": a step's byte floor is its weight bytes over the memory
 * bandwidth). sink: a device uint32 that is written only if the xor of all the data read equals
 * 0x9E3779B9 (it keeps the loads from being dropped). a, b 16-byte aligned; a_bytes, b_bytes >= 0
 * and multiples of 16, a_bytes + b_bytes below 63 GiB (b may be NULL when b_bytes == 0). Errors:
 * ATTNQ_ERR_NULL, ATTNQ_ERR_SHAPE, ATTNQ_ERR_ALIGN, ATTNQ_ERR_HIP. */
ATTNQ_API attnq_status attnq_read_ceiling(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes,
                                uint32_t* sink, attnq_stream stream);

/* Static string naming a status code (host only). */
ATTNQ_API const char* attnq_status_string(attnq_status status);

#ifdef __cplusplus
}
#endif

#endif /* ATTNQ_H */
