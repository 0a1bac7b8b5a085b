/*
 * weight_only_bit -- MI355X (gfx950) weight-only 4-bit GEMM library, C ABI.
 *
 *     Y[M,N] = X[M,K] . dequant(Wq)[N,K]^T
 *
 * Two weight formats:
 *  - W4A16: unsigned 4-bit codes q, a scale s per (row, group of g along K) in
 *    the activation dtype and an unsigned 4-bit zero-point z per (row, group);
 *    w = (q - z) * s.  Source: "Keep W4A16 zero-points packed at 4 bits instead
 *    of expanding to 2 bytes" (ROCm/vllm pull request 1073), sections Problem
 *    and Change: the skinny W4A16 GEMM takes the zero-points packed eight per
 *    int32 along N and extracts the nibble of row n from word n/8 at bits
 *    4*(n%8); activation-dtype zero-points are rejected rather than
 *    reinterpreted (section Testing).
 *  - MXFP4 (OCP MX E2M1 elements, one E8M0 scale per 32 along K) for MoE
 *    stage 1 with BF16 activations.  Source: "Add BF16xFP4 MoE GEMM stage1
 *    kernel" (ROCm/FlyDSL pull request 424), summary and Technical Details: the
 *    FP4 weights are dequantized to BF16 in software (one scaled conversion per
 *    byte, two elements each) before each BF16 matrix-core multiply; the E8M0
 *    byte is the binary32 exponent of the scale; the store guard keeps
 *    out-of-range tiles from writing into neighbouring token-slot rows.
 *
 * Layouts (all row-major, contiguous, device memory unless stated):
 *   x        [M][K]        activation dtype (WOB_F16 or WOB_BF16)
 *   qweight  [N][K/8]      int32; code of (n, k) is bits 4*(k%8) of word (n, k/8)
 *   scales   [N][K/g]      activation dtype (must equal x's dtype)
 *   qzeros   [N/8][K/g]    int32; zero-point of (n, j) is bits 4*(n%8) of word (n/8, j)
 *                          NULL means symmetric codes: z = 8 for every group
 *   y        [M][N]        activation dtype, rounded to nearest even from fp32
 *   w_fp4    [E][N][K/2]   uint8; element k is the low nibble of byte k/2 when
 *                          k is even, the high nibble when k is odd
 *   w_scale  [E][N][K/32]  uint8 E8M0 exponent b; scale = 2^(b-127) for every
 *                          b in 0..254 (b = 0 is 2^-127), NaN for b = 255
 *                          (OCP MX E8M0)
 * Packed words are unsigned bit containers (logical shifts).
 *
 * Conventions shared by every entry point:
 *  - All pointers are owned by the caller; the library keeps no allocation and
 *    no state beyond a per-device architecture check and the per-device LDS
 *    limit of its large-tile kernels (set on first use).
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *    void*, NULL = the null stream) for the calling thread's current HIP
 *    device, which the stream and every pointer must belong to; nothing
 *    synchronizes.
 *  - Every argument is validated before any device call; on a non-zero status
 *    nothing was enqueued.  No exception crosses the ABI.
 *  - Device pointers must be 16-byte aligned.
 *  - Results are deterministic for a fixed shape: the summation order over K
 *    does not depend on timing.
 */
#ifndef WEIGHT_ONLY_BIT_H
#define WEIGHT_ONLY_BIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define WOB_OK 0
#define WOB_INVALID_ARG 1 /* null pointer, bad shape, misalignment, small workspace */
#define WOB_DTYPE 2       /* a dtype tag the operand cannot have (e.g. act-dtype zero-points) */
#define WOB_UNSUPPORTED 3 /* device is not gfx950, or a group size the kernels do not take */
#define WOB_HIP 4         /* the HIP runtime reported an error at launch */

/* Dtype tags. */
#define WOB_F16 0
#define WOB_BF16 1
#define WOB_U4X8_I32 2 /* eight 4-bit values packed in an int32 */
#define WOB_F32 3

/* MoE stage-1 activation (the `act` argument of mxfp4_moe_gemm). */
#define WOB_ACT_NONE 0     /* pre-activation output [T][topk][N] */
#define WOB_ACT_SILU_MUL 1 /* silu(gate) * up: output [T][topk][N/2] */

/* Kernel path selection for w4a16_gemm_ex. */
#define WOB_PATH_AUTO 0   /* M <= 8 (and X fits the skinny kernel's LDS) -> skinny, else tiled */
#define WOB_PATH_SKINNY 1 /* split-K GEMV; requires M <= 8 */
#define WOB_PATH_TILED 2  /* cooperative-tile MFMA GEMM; any M >= 1 */

/* Text of a status code (static storage). */
const char *wob_status_str(int status);

/* Detail of the last non-OK status returned on this thread (static/thread-local storage). */
const char *wob_last_error(void);

/*
 * Check that the current HIP device is gfx950.  Returns WOB_OK or
 * WOB_UNSUPPORTED (WOB_HIP if the runtime cannot be queried).
 */
int wob_device_check(void);

/*
 * W4A16 GEMM: y[m][n] = sum_k x[m][k] * (q(n,k) - z(n,k/g)) * s(n,k/g).
 * Source: zero-point page above, sections Problem and Change (packed
 * zero-points, nibble extraction inside the kernel).
 *
 *  x_dtype, scales_dtype: WOB_F16 or WOB_BF16 and equal, else WOB_DTYPE.
 *  zeros_dtype: WOB_U4X8_I32 (ignored when qzeros == NULL); any other tag
 *    -> WOB_DTYPE (activation-dtype zero-points are refused, not reinterpreted).
 *  group_size in {32, 64, 128} (else WOB_UNSUPPORTED); K % group_size == 0,
 *    K % 32 == 0, N % 8 == 0, M >= 0, N >= 0, K >= 32, N*K/2 below 2^32
 *    (else WOB_INVALID_ARG).  When the tiled path runs (M > 8, or the skinny
 *    kernel's LDS cannot hold M*K activations), also 2*K*min(M, 256) below
 *    2^32 (else WOB_INVALID_ARG).
 *    M == 0 or N == 0 is a no-op returning WOB_OK.
 *  Arithmetic, fp32 accumulation in both paths: the skinny path (M <= 8)
 *  multiplies x with the exact (q - z) (exact products) and scales each
 *  32-wide chunk's sum by s; the tiled path multiplies x with (q - z) * s
 *  rounded once to x's dtype.  y is rounded to nearest even in x's dtype.
 */
int w4a16_gemm(const void *x, int x_dtype, const int32_t *qweight, const void *scales,
               int scales_dtype, const void *qzeros, int zeros_dtype, void *y, int64_t M,
               int64_t N, int64_t K, int64_t group_size, void *stream);

/* As w4a16_gemm with an explicit kernel path (WOB_PATH_*); WOB_PATH_SKINNY
 * with M > 8 or M*K too large for the skinny kernel's LDS gives
 * WOB_INVALID_ARG.  Not part of the method: it lets tests and measurements
 * run each kernel on the same inputs. */
int w4a16_gemm_ex(const void *x, int x_dtype, const int32_t *qweight, const void *scales,
                  int scales_dtype, const void *qzeros, int zeros_dtype, void *y, int64_t M,
                  int64_t N, int64_t K, int64_t group_size, int path, void *stream);

/*
 * Ragged grouped W4A16 GEMM ("contiguous grouped" form): group e owns rows
 * [m_offsets[e], m_offsets[e+1]) of x[total_M][K] and y[total_M][N] and uses
 * its own weights qweight[e][N][K/8], scales[e][N][K/g], qzeros[e][N/8][K/g]
 * (qzeros may be NULL: symmetric).  m_offsets is a DEVICE int64 array of
 * num_groups+1 entries that must be nondecreasing from 0 to total_M (a
 * precondition; the kernel clamps every range to [0, total_M]).  Rows outside
 * every group are not written.  Same dtype and shape rules as w4a16_gemm.
 * Source: the grouped GEMM named on "ROCm IQ4_XS keep-quant GEMM is 8.8x
 * behind llama.cpp's WMMA path" (vllm.cpp issue 3006), section What already
 * exists; the ragged-offset reading is this library's.  The tiled path's
 * bound 2*K*min(total_M, 256) below 2^32 applies.
 */
int w4a16_gemm_grouped(const void *x, int x_dtype, const int64_t *m_offsets, int64_t num_groups,
                       int64_t total_M, const int32_t *qweight, const void *scales,
                       int scales_dtype, const void *qzeros, int zeros_dtype, void *y, int64_t N,
                       int64_t K, int64_t group_size, void *stream);

/*
 * Bytes of device workspace mxfp4_moe_gemm needs for T tokens, topk slots, E
 * experts (routing scratch: per-expert tiles and the pairs sorted by expert;
 * N and K do not change it).  0 for arguments mxfp4_moe_gemm would refuse
 * (T < 0, topk outside 1..64, E outside 1..4096, N or K negative).
 */
size_t mxfp4_moe_gemm_workspace_size(int64_t T, int64_t topk, int64_t E, int64_t N, int64_t K);

/*
 * MoE stage 1, BF16 x MXFP4: for token t and slot s with expert e = topk_ids[t][s],
 *   pre[t][s][n] = sum_k x[t][k] * e2m1(code_e(n,k)) * 2^(w_scale[e][n][k/32] - 127)
 * (gate and up halves of N as stored; no routing-weight multiply).
 * Source: MXFP4 page above, summary and Technical Details.
 *
 *  act == WOB_ACT_NONE: y [T][topk][N] bf16 = pre.
 *  act == WOB_ACT_SILU_MUL: the N rows of each expert's W1 are a gate half
 *    (rows 0 .. N/2-1) and an up half (rows N/2 .. N-1), and
 *      y[t][s][n] = silu(g) * u,  g = pre[t][s][n], u = pre[t][s][N/2 + n],
 *      silu(v) = v / (1 + e^-v),  n < N/2,
 *    into y [T][topk][N/2] bf16 (pre stays in fp32 and is never written).
 *    Source: MXFP4 page above, summary and Test (the stage-1 kernel's silu
 *    activation; the gate/up split of W1 is this library's reading).
 *    Needs N % 32 == 0.  Any other act gives WOB_INVALID_ARG.
 *
 *  x [T][K] bf16; topk_ids [T][topk] int32 on the device.
 *  Rows whose id lies outside [0, E) are written as zeros.
 *  K % 64 == 0 (the page's 64-wide K tile), K >= 64, N % 16 == 0, T >= 0,
 *  1 <= topk <= 64, 1 <= E <= 4096, T*K*2 and N*K/2 below 2^32 (else
 *  WOB_INVALID_ARG).
 *  workspace: device memory of at least mxfp4_moe_gemm_workspace_size(T, topk,
 *  E, N, K) bytes, 16-byte aligned (else WOB_INVALID_ARG); its contents on
 *  entry do not matter.  Calls that share one workspace must be ordered on
 *  one stream.  Decode batches (T <= 8, with K <= 32768) run a memory-bound
 *  kernel that routes on its own and leaves the workspace untouched; the
 *  workspace is still required and checked.  Both kernels compute the same
 *  function.
 */
int mxfp4_moe_gemm(const void *x, const int32_t *topk_ids, const uint8_t *w_fp4,
                   const uint8_t *w_scale, void *y, int64_t T, int64_t topk, int64_t E, int64_t N,
                   int64_t K, int act, void *workspace, size_t workspace_bytes, void *stream);

/*
 * mxfp4_moe_gemm with a chosen tile height tile_m: each expert's routed rows
 * are padded to a multiple of tile_m (the MFMA block height of the expert
 * tiles), 16 or 32 (else WOB_INVALID_ARG).  Source: MXFP4 page above, Test
 * Plan / Test Result (the stage-1 kernel is built and tested per tile height).
 * mxfp4_moe_gemm is tile_m = 32.  Same function, arguments, workspace and
 * errors; decode batches (T <= 8) take the memory-bound kernel whatever
 * tile_m is.  16 wastes fewer products on padding but measures slower on
 * MI355X at every batch size tried (16 to 1024 tokens).
 */
int mxfp4_moe_gemm_tile_m(const void *x, const int32_t *topk_ids, const uint8_t *w_fp4,
                          const uint8_t *w_scale, void *y, int64_t T, int64_t topk, int64_t E,
                          int64_t N, int64_t K, int act, int tile_m, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * Bytes of device workspace mxfp4_moe_stage2 needs: the routing scratch of
 * stage 1 plus T*topk*H fp32 per-pair results.  0 for arguments it refuses
 * on sight (T < 0, topk outside 1..64, E outside 1..4096, H or I negative).
 */
size_t mxfp4_moe_stage2_workspace_size(int64_t T, int64_t topk, int64_t E, int64_t H, int64_t I);

/*
 * MoE stage 2, BF16 x MXFP4: the down projection of the stage-1 activation
 * rows with the routing-weight combine,
 *   y[t][h] = sum over s < topk with e = topk_ids[t][s] in [0, E) of
 *             topk_weights[t][s] * sum_i a[t][s][i] * w2_e(h, i),
 *   w2_e(h, i) = e2m1(code) * 2^(w2_scale[e][h][i/32] - 127) as in stage 1.
 * The MXFP4 page above names its kernel stage 1 (summary, Test); the second
 * stage is this library's reading of the MoE layer it belongs to: each
 * routed row of the stage-1 output (act == WOB_ACT_SILU_MUL, I = N/2) is
 * multiplied with its expert's W2, weighted, and the token's slots summed.
 *
 *  a [T][topk][I] bf16; topk_ids [T][topk] int32 (device, as for stage 1);
 *  topk_weights [T][topk] fp32 (device); w2_fp4 [E][H][I/2] uint8 (even i in
 *  the low nibble); w2_scale [E][H][I/32] uint8 E8M0; y [T][H] bf16.
 *  Slots whose id lies outside [0, E) contribute nothing.  Each slot's
 *  products accumulate in fp32; the weighted slots are summed in slot order
 *  in fp32 and rounded once to bf16 (deterministic).
 *  I % 64 == 0, I >= 64, H % 16 == 0, T >= 0, 1 <= topk <= 64,
 *  1 <= E <= 4096, T*topk*I*2 and H*I/2 below 2^32 (else WOB_INVALID_ARG).
 *  T == 0 or H == 0 is a no-op returning WOB_OK.
 *  workspace: device memory of at least mxfp4_moe_stage2_workspace_size(T,
 *  topk, E, H, I) bytes, 16-byte aligned; contents on entry do not matter.
 *  Calls sharing one workspace must be ordered on one stream.
 */
int mxfp4_moe_stage2(const void *a, const int32_t *topk_ids, const float *topk_weights,
                     const uint8_t *w2_fp4, const uint8_t *w2_scale, void *y, int64_t T,
                     int64_t topk, int64_t E, int64_t H, int64_t I, void *workspace,
                     size_t workspace_bytes, void *stream);

/*
 * mxfp4_moe_gemm without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the routing scratch lives in a static
 * device array of 1 MiB (one per GPU, held until the process ends).  Same
 * operands, rules, kernels and results as mxfp4_moe_gemm; additionally
 * mxfp4_moe_gemm_workspace_size(T, topk, E, N, K) must not exceed 1 MiB
 * (about 250,000 routed pairs T*topk at E = 32), else WOB_INVALID_ARG before
 * any device call.  Every call on one GPU uses that GPU's one array, so calls
 * that overlap on one GPU (concurrent streams or threads) race; calls ordered
 * on one stream do not.  The array needs no clearing: each call rewrites what
 * it reads.  Allocates nothing (no hipMalloc, hipFree or allocating library
 * call); the array's device address is looked up once per device.
 */
int mxfp4_moe_gemm_noalloc(const void *x, const int32_t *topk_ids, const uint8_t *w_fp4,
                           const uint8_t *w_scale, void *y, int64_t T, int64_t topk, int64_t E,
                           int64_t N, int64_t K, int act, void *stream);

/*
 * Dequantization probes: write out the weights as the GEMM kernels form them,
 * through the same device helpers, so the unpack / dequantize stage can be
 * compared bit for bit with its definition.  Source: zero-point page above,
 * section Testing (value-level checks against a reference dequantization, so
 * that a wrong nibble index cannot pass silently).
 *  out_dtype WOB_F32: the skinny kernel's exact (q - z), formed by that
 *    kernel's helpers, times the scale in fp32 (exact; the kernel itself
 *    applies the scale to each 32-wide chunk's sum of products).
 *  out_dtype == scales_dtype: the tiled kernels' MFMA operand values,
 *    (q - z) * s rounded to nearest even in that dtype.
 * Same shape and dtype rules as w4a16_gemm (zeros_dtype, here too, must be
 * WOB_U4X8_I32 when qzeros is given).
 */
int w4a16_dequant(const int32_t *qweight, const void *scales, int scales_dtype,
                  const void *qzeros, int zeros_dtype, void *out, int out_dtype, int64_t N,
                  int64_t K, int64_t group_size, void *stream);

/*
 * MXFP4 probe: out[N][K] bf16 = the MoE kernels' weight-operand values for
 * one expert (E2M1 code times the E8M0 scale, as v_cvt_scalef32_pk_bf16_fp4
 * forms them).  Source: MXFP4 page above, Technical Details.  K % 32 == 0,
 * K >= 32, N >= 0, w_fp4 and out 16-byte aligned (else WOB_INVALID_ARG).
 */
int mxfp4_dequant(const uint8_t *w_fp4, const uint8_t *w_scale, void *out, int64_t N, int64_t K,
                  void *stream);

/*
 * Streaming-read reference (a measurement aid, not part of the method): reads
 * the `bytes` bytes at `buf` once with 16-byte loads, as fast as a kernel that
 * only reads can, so that the GEMV kernels' rates can be compared with the
 * device's own streaming rate for the same byte count.  bytes % 16 == 0;
 * `buf` 16-byte aligned; `sink` is device memory of at least 1024 bytes that
 * the call may overwrite (its contents carry no meaning).  bytes == 0 is a
 * no-op.  Errors as for the entry points above.
 */
int wob_stream_read(const void *buf, size_t bytes, void *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* WEIGHT_ONLY_BIT_H */
