/*
 * fp4blk.h -- C ABI of libfp4blk: block-scaled 4-bit (NVFP4, MXFP4)
 * quantization and the quantized linear-layer GEMMs it feeds, for AMD
 * Instinct MI355X (gfx950).
 *
 * Formats (pages cited by title and section):
 *  - NVFP4: "NVFP4" (newton.com.tw wiki), section "Technical principle".
 *    E2M1 elements (1 sign, 2 exponent, 1 mantissa bit; values
 *    {0, 0.5, 1, 1.5, 2, 3, 4, 6} and their negatives), 16-element micro-blocks
 *    each with one E4M3 (OCP E4M3FN: bias 7, largest 448, no infinities) scale
 *    byte, and one FP32 scale per tensor: 4.5 bits per value.
 *  - MXFP4: edge-FP4 article (eefocus.com), section "FP4 as the next core
 *    standard".  OCP MX block floating point: 32-element blocks, one E8M0 byte
 *    (2^(byte-127)) per block, E2M1 elements: 4.25 bits per value.
 *  - W4A16 / W4A4: Unsloth Dynamic NVFP4 article (aixq.cc), section "Core
 *    difference: W4A4 vs W4A16".  W4A16 multiplies 4-bit weights, widened to
 *    16 bits, by 16-bit activations; W4A4 quantizes the activations to 4 bits
 *    as well.
 *
 * Packed layout (every packed tensor, row-major, blocks along the last axis):
 *  - codes  uint8 [rows][cols/2]: element (r, c) is in byte r*cols/2 + c/2, in
 *           the low nibble when c is even and the high nibble when c is odd;
 *           nibble = sign<<3 | magnitude index into the grid above.
 *  - scales uint8 [rows][cols/16] (NVFP4, E4M3FN bytes) or [rows][cols/32]
 *           (MXFP4, E8M0 bytes).
 *  - tscale float32 [1] (per tensor) or [rows] (per row): the NVFP4 second-level
 *           scale; value = E2M1(code) * E4M3(scale byte) * tscale.
 * A GEMM computes C[m][n] = sum_k A[m][k] * W[n][k] (C = A . W^T) with W [N][K]
 * packed as above and blocks running along K.
 *
 * Quantization recipe (NVFP4):
 *   tscale    = fl32(amax / 2688)                      (2688 = 6 * 448)
 *   scale[b]  = E4M3 round-to-nearest-even, saturating at 448, of
 *               fl32(block_amax / fl32(6 * tscale)); 0x00 for an all-zero block
 *   code      = E2M1 round-to-nearest-even (ties to the even mantissa bit),
 *               saturating at 6, of fl32(x / fl32(E4M3(scale[b]) * tscale));
 *               a signed zero when that divisor is zero
 * MXFP4: k = floor(log2 block_amax) - 2 (FP4_MX_OCP_FLOOR) or the smallest k
 * with 6 * 2^k >= block_amax (FP4_MX_CEIL), clamped to [-127, 127]; scale byte
 * k + 127 (0 for an all-zero block); code = E2M1-RNE-saturating(x * 2^-k).
 *
 * Conventions:
 *  - Every data pointer is a DEVICE pointer owned by the caller.  The library
 *    allocates and frees nothing.  Its only global state is per-device and
 *    written once per device with atomics (whether the device is a gfx950, its
 *    CU count, which kernels had their LDS limit raised, the device address of
 *    the scratch array of gemm_w4a4_noalloc), plus that scratch array itself;
 *    calls are thread-safe, except that calls of gemm_w4a4_noalloc that
 *    overlap on one device share its scratch.
 *  - Every call is asynchronous on `stream` (0 = the null stream) and never
 *    synchronizes the host.
 *  - Arguments are validated on the host before anything is launched; on an
 *    error nothing is launched and the outputs are untouched.  Validation:
 *    non-null pointers, all sizes > 0, leading dimensions >= the row length,
 *    cols (or K) a multiple of 16 (NVFP4) / 32 (MXFP4), 16-byte aligned base
 *    pointers and leading dimensions that keep every row 16-byte aligned,
 *    workspace at least the queried size.
 *  - Launch failures return FP4_ERR_HIP.  Non-finite inputs (NaN, Inf) violate
 *    a precondition: outputs are unspecified and, if `nonfinite` is non-null,
 *    the device int it points to is set to 1 (it is never cleared by the
 *    library).
 *  - No C++ exception crosses this interface.
 */
#ifndef FP4BLK_H
#define FP4BLK_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FP4_OK = 0,
    FP4_ERR_NULL = 1,               /* a required pointer is null */
    FP4_ERR_SHAPE = 2,              /* a size is <= 0, or not a whole number of blocks */
    FP4_ERR_LAYOUT = 3,             /* leading dimension too small, or misaligned pointer/row */
    FP4_ERR_DTYPE = 4,              /* unknown dtype / mode / rule value */
    FP4_ERR_WORKSPACE = 5,          /* workspace null or smaller than the queried size */
    FP4_ERR_NO_DEVICE = 6,          /* no HIP device is visible */
    FP4_ERR_UNSUPPORTED_DEVICE = 7, /* the current device is not gfx950 */
    FP4_ERR_HIP = 8                 /* a HIP call or kernel launch failed */
} fp4_status;

typedef enum { FP4_F32 = 0, FP4_BF16 = 1 } fp4_dtype;
typedef enum { FP4_SCALE_PER_TENSOR = 0, FP4_SCALE_PER_ROW = 1 } fp4_scale_mode;
typedef enum { FP4_MX_OCP_FLOOR = 0, FP4_MX_CEIL = 1 } fp4_mx_rule;

/* Human-readable name of a status code (static string; never null). */
const char *fp4_status_str(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int fp4blk_version(void);

/* FP4_OK if the current HIP device is a gfx950, else NO_DEVICE / UNSUPPORTED_DEVICE. */
fp4_status fp4blk_check_device(void);

/* ------------------------------------------------------------ NVFP4 ------ */

/* Workspace bytes nvfp4_quantize needs (0 for FP4_SCALE_PER_ROW). */
size_t nvfp4_quantize_workspace(int64_t rows, int64_t cols, fp4_scale_mode mode);

/* NVFP4 quantize ("NVFP4", Technical principle: two-level micro-block scaling).
 *  x        [rows][ldx] fp32 or bf16 (xt), cols % 16 == 0, read only.
 *  codes    [rows][cols/2] out; scales [rows][cols/16] out (E4M3FN bytes).
 *  tscale   out: [1] for FP4_SCALE_PER_TENSOR (amax over the whole tensor),
 *           [rows] for FP4_SCALE_PER_ROW (each row is its own tensor).
 *  ws       device scratch of nvfp4_quantize_workspace() bytes (per-tensor mode).
 *  nonfinite optional device int32 flag, set to 1 if x holds NaN/Inf.
 * Codes and scale bytes equal the recipe above bit for bit. */
fp4_status nvfp4_quantize(const void *x, fp4_dtype xt, int64_t rows, int64_t cols, int64_t ldx,
                          uint8_t *codes, uint8_t *scales, float *tscale, fp4_scale_mode mode,
                          void *ws, size_t ws_bytes, int32_t *nonfinite, hipStream_t stream);

/* NVFP4 dequantize ("NVFP4", Technical principle: a value is its E2M1 element
 * times its micro-block's E4M3 scale times the FP32 tensor scale; the W4A16
 * path of the aixq.cc article, "Core difference: W4A4 vs W4A16", restores the
 * weights to 16 bits this way):
 *  y = fl32(fl32(E2M1(c) * E4M3(s)) * tscale) (the inner product is exact),
 *  stored as fp32 or rounded to nearest even into bf16 (yt).
 *  codes [rows][cols/2], scales [rows][cols/16], tscale [1] (FP4_SCALE_PER_TENSOR)
 *  or [rows] (FP4_SCALE_PER_ROW): device, read only.  cols % 16 == 0.
 *  y [rows][ldy] out (ldy >= cols, 16-byte aligned rows), caller-owned.
 * Errors (host, nothing launched): FP4_ERR_NULL, FP4_ERR_SHAPE, FP4_ERR_LAYOUT,
 * FP4_ERR_DTYPE as for nvfp4_quantize. */
fp4_status nvfp4_dequantize(const uint8_t *codes, const uint8_t *scales, const float *tscale,
                            fp4_scale_mode mode, int64_t rows, int64_t cols, void *y,
                            fp4_dtype yt, int64_t ldy, hipStream_t stream);

/* W4A16 GEMM (aixq.cc article, "Core difference: W4A4 vs W4A16"): C = A . W^T.
 *  a        [M][lda] bf16 activations.
 *  w_*      W [N][K] NVFP4 with a per-tensor scale (w_tscale[1]).
 *  c        [M][ldc] out, fp32 or bf16 (ct; bf16 by round to nearest even).
 * Each weight is widened exactly to E2M1 * E4M3 in bfloat16, products are
 * accumulated in fp32 and the sum is multiplied by w_tscale.  |C - C_exact|
 * stays within 2e-3 * sum_k |a w| (C_exact: fp64 over the dequantized W). */
fp4_status gemm_w4a16(const void *a, int64_t M, int64_t K, int64_t lda, const uint8_t *w_codes,
                      const uint8_t *w_scales, const float *w_tscale, int64_t N, void *c,
                      fp4_dtype ct, int64_t ldc, hipStream_t stream);

/* Decode layout of an NVFP4 weight (for gemm_w4a16_decode).  K is cut into
 * 128-element segments; the layout stores them segment-major,
 *   codes_p  uint8 [K/128][N][64]: byte (s*N + n)*64 + b = codes[n][64*s + b]
 *   scales_p uint8 [K/128][N][8]:  byte (s*N + n)*8 + b  = scales[n][8*s + b]
 * so the 16 rows of a matrix-core tile at one segment are 1 KiB of
 * consecutive bytes.  Same bytes and byte count as the row-major form (4.5 bits
 * a value); only the order differs.  The tensor scale is unchanged.
 * nvfp4_pack_decode rewrites row-major codes [N][K/2] / scales [N][K/16] into
 * it (K % 128 == 0; outputs of N*K/2 and N*K/16 bytes, not overlapping the
 * inputs). */
fp4_status nvfp4_pack_decode(const uint8_t *codes, const uint8_t *scales, int64_t N, int64_t K,
                             uint8_t *codes_p, uint8_t *scales_p, hipStream_t stream);

/* W4A16 (aixq.cc article, "Core difference: W4A4 vs W4A16") on a weight in the
 * decode layout: C = A . W^T, K % 128 == 0.  1 <= M <= 16 (any such K) runs the
 * decode GEMV; larger M the prefill GEMM reading the same layout (the result
 * gemm_w4a16 gives on the row-major weight, bit for bit), so one packed weight
 * serves both.  Same arithmetic and tolerance as gemm_w4a16 (each weight widened
 * exactly to E2M1 * E4M3 in bfloat16, fp32 accumulation, times w_tscale).
 * FP4_ERR_SHAPE, checked on the host before anything is launched, for any M
 * when A spans 2 GiB or more (M * lda * 2 or (M - 1) * lda * 2 + 2 K bytes) or
 * the weight codes do (N * K / 2 bytes): both kernels address the operands with
 * 32-bit byte offsets. */
fp4_status gemm_w4a16_decode(const void *a, int64_t M, int64_t K, int64_t lda, const uint8_t *w_codes_p,
                             const uint8_t *w_scales_p, const float *w_tscale, int64_t N, void *c,
                             fp4_dtype ct, int64_t ldc, hipStream_t stream);

/* Workspace bytes gemm_w4a4 needs: A's codes | scales | tscale, each starting
 * at a 256-byte boundary, in that order (offsets by gemm_w4a4_workspace_offsets). */
size_t gemm_w4a4_workspace(int64_t M, int64_t K, fp4_scale_mode a_mode);
void gemm_w4a4_workspace_offsets(int64_t M, int64_t K, size_t *codes_off, size_t *scales_off,
                                 size_t *tscale_off);

/* W4A4 NVFP4 GEMM (aixq.cc article, "Core difference"): the bf16 activations
 * are quantized to NVFP4 on the device (a_mode: per row, each row its own
 * tensor, or per tensor) into `ws`, then C = A_q . W^T with both operands
 * widened exactly to bfloat16, fp32 accumulation, and the epilogue multiplies
 * by the activation scale (per row) and the weight tensor scale.  After the call
 * `ws` holds A's packed NVFP4 form (codes, scales, tscale) at the documented
 * offsets.  Same tolerance as gemm_w4a16, against fp64 over the two dequantized
 * operands. */
fp4_status gemm_w4a4(const void *a, int64_t M, int64_t K, int64_t lda, fp4_scale_mode a_mode,
                     const uint8_t *w_codes, const uint8_t *w_scales, const float *w_tscale,
                     int64_t N, void *c, fp4_dtype ct, int64_t ldc, void *ws, size_t ws_bytes,
                     hipStream_t stream);

/* The GEMM half of gemm_w4a4 on an already-quantized A (codes [M][K/2],
 * scales [M][K/16], a_tscale [1] or [M] per a_mode). */
fp4_status gemm_nvfp4_w4a4_prequant(const uint8_t *a_codes, const uint8_t *a_scales,
                                    const float *a_tscale, fp4_scale_mode a_mode, int64_t M,
                                    int64_t K, const uint8_t *w_codes, const uint8_t *w_scales,
                                    const float *w_tscale, int64_t N, void *c, fp4_dtype ct,
                                    int64_t ldc, hipStream_t stream);

/* NVFP4 W4A4 with W in the decode layout (nvfp4_pack_decode): the same result as
 * gemm_w4a4 / gemm_nvfp4_w4a4_prequant on the row-major W, bit for bit; each
 * 64-element K stage then reads a weight panel whose rows are 64 bytes apart
 * instead of K/2.  K % 128 == 0, M * K / 2 and N * K / 2 below 2^31
 * (FP4_ERR_SHAPE otherwise, checked before A is quantized); other arguments,
 * workspace and errors as those two. */
fp4_status gemm_w4a4_seg(const void *a, int64_t M, int64_t K, int64_t lda, fp4_scale_mode a_mode,
                         const uint8_t *w_codes_p, const uint8_t *w_scales_p, const float *w_tscale, int64_t N,
                         void *c, fp4_dtype ct, int64_t ldc, void *ws, size_t ws_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): gemm_w4a4 with A's
 * packed NVFP4 form kept in the library's own device scratch instead of a
 * caller's workspace.  The scratch is 32 MiB (33,554,432 bytes) per device, held
 * from the time the library's code is loaded on the device until the process
 * ends.  Arguments as gemm_w4a4 without ws / ws_bytes (W row-major); the result
 * is gemm_w4a4's, bit for bit.  FP4_ERR_WORKSPACE when gemm_w4a4_workspace(M, K,
 * a_mode) exceeds 32 MiB (M * K up to about 29.6 million with per-row scales),
 * checked on the host before anything is launched; other errors as gemm_w4a4.
 * The call allocates and frees nothing.  Every call on a device uses that
 * device's one scratch: calls that overlap on one device (two streams, or two
 * host threads without ordering) race and give unspecified results; calls
 * ordered on one stream do not.  A's packed form stays in the scratch until the
 * next call, but its address is not part of this interface. */
fp4_status gemm_w4a4_noalloc(const void *a, int64_t M, int64_t K, int64_t lda, fp4_scale_mode a_mode,
                             const uint8_t *w_codes, const uint8_t *w_scales, const float *w_tscale, int64_t N,
                             void *c, fp4_dtype ct, int64_t ldc, hipStream_t stream);
fp4_status gemm_nvfp4_w4a4_prequant_seg(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_tscale,
                                        fp4_scale_mode a_mode, int64_t M, int64_t K, const uint8_t *w_codes_p,
                                        const uint8_t *w_scales_p, const float *w_tscale, int64_t N, void *c,
                                        fp4_dtype ct, int64_t ldc, hipStream_t stream);

/* ------------------------------------------------------------ MXFP4 ------ */

/* MXFP4 quantize (eefocus.com article, "FP4 as the next core standard").
 *  x [rows][ldx] fp32 or bf16, cols % 32 == 0; codes [rows][cols/2] out;
 *  scales [rows][cols/32] E8M0 out; rule FP4_MX_OCP_FLOOR or FP4_MX_CEIL. */
fp4_status mxfp4_quantize(const void *x, fp4_dtype xt, int64_t rows, int64_t cols, int64_t ldx,
                          uint8_t *codes, uint8_t *scales, fp4_mx_rule rule, int32_t *nonfinite,
                          hipStream_t stream);

/* MXFP4 dequantize (eefocus.com edge-FP4 article, "FP4 as the next core
 * standard": each 32-element block shares one E8M0 power-of-two scale):
 *  y = E2M1(c) * 2^(s-127) (exact when in range), fp32, or bf16 by round to
 *  nearest even; the scale byte 0xFF (E8M0's NaN) gives NaN for its block.  codes [rows][cols/2], scales [rows][cols/32]: device, read
 *  only; cols % 32 == 0.  y [rows][ldy] out (ldy >= cols, 16-byte aligned rows).
 * Errors (host, nothing launched): FP4_ERR_NULL, FP4_ERR_SHAPE, FP4_ERR_LAYOUT,
 * FP4_ERR_DTYPE. */
fp4_status mxfp4_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t rows,
                            int64_t cols, void *y, fp4_dtype yt, int64_t ldy, hipStream_t stream);

/* Workspace bytes mxfp4_gemm_w4a4 needs: A's codes | scales, 256-byte aligned. */
size_t mxfp4_gemm_w4a4_workspace(int64_t M, int64_t K);

/* 1 if mxfp4_gemm_w4a4 leaves A's MXFP4 form in its workspace segment-major
 * (codes [K/128][M][64], E8M0 [K/128][M][4], as mxfp4_gemm_w4a4_seg does): when
 * K % 128 == 0 and A's and W's codes are each under 2 GiB.  0: row-major
 * (codes [M][K/2], E8M0 [M][K/32]).  Either way the bytes are those of
 * mxfp4_quantize(A); only their order differs. */
int mxfp4_gemm_w4a4_a_segment_major(int64_t M, int64_t N, int64_t K);

/* MXFP4 W4A4 GEMM: A (bf16) is quantized to MXFP4 with `rule` into `ws`, then
 * C = A_q . W^T on gfx950's block-scaled FP4 matrix instruction (E8M0 scale per
 * 32 K-elements per row, the MX block), fp32 accumulation.  W [N][K] MXFP4.
 * A's form in `ws` is segment-major where mxfp4_gemm_w4a4_a_segment_major says
 * so (the kernel then reads W's 64-byte row pieces per 128-K segment, A's
 * panels as contiguous runs); the result is the same bit for bit. */
fp4_status mxfp4_gemm_w4a4(const void *a, int64_t M, int64_t K, int64_t lda, fp4_mx_rule rule,
                           const uint8_t *w_codes, const uint8_t *w_scales, int64_t N, void *c,
                           fp4_dtype ct, int64_t ldc, void *ws, size_t ws_bytes,
                           hipStream_t stream);

/* The GEMM half of mxfp4_gemm_w4a4 on an already-quantized A. */
fp4_status mxfp4_gemm_prequant(const uint8_t *a_codes, const uint8_t *a_scales, int64_t M,
                               int64_t K, const uint8_t *w_codes, const uint8_t *w_scales,
                               int64_t N, void *c, fp4_dtype ct, int64_t ldc, hipStream_t stream);

/* MXFP4 W4A16 GEMM (eefocus.com edge-FP4 article, "FP4 as the next core
 * standard": MXFP4 blocks of 32 elements with an E8M0 power-of-two scale; aixq.cc
 * article, "Core difference: W4A4 vs W4A16": 16-bit activations): C = A . W^T
 * with A bf16 [M][lda] and W MXFP4 row-major, codes [N][K/2], E8M0 scales
 * [N][K/32].  Each weight is widened exactly to bf16 (E2M1 times a power of two),
 * fp32 accumulation; no tensor scale.  K % 128 == 0 (FP4_ERR_SHAPE otherwise, and
 * for operands past 2 GiB).  Tolerance as gemm_w4a16. */
fp4_status mxfp4_gemm_w4a16(const void *a, int64_t M, int64_t K, int64_t lda, const uint8_t *w_codes,
                            const uint8_t *w_scales, int64_t N, void *c, fp4_dtype ct, int64_t ldc,
                            hipStream_t stream);

/* Decode layout of an MXFP4 weight: codes as for nvfp4_pack_decode,
 *   codes_p  uint8 [K/128][N][64]: byte (s*N + n)*64 + b = codes[n][64*s + b]
 *   scales_p uint8 [K/128][N][4]:  byte (s*N + n)*4 + b  = scales[n][4*s + b]
 * (the 4 E8M0 bytes of segment s).  Same bytes and count as the row-major form
 * (4.25 bits a value).  K % 128 == 0; outputs of N*K/2 and N*K/32 bytes, not
 * overlapping the inputs. */
fp4_status mxfp4_pack_decode(const uint8_t *codes, const uint8_t *scales, int64_t N, int64_t K,
                             uint8_t *codes_p, uint8_t *scales_p, hipStream_t stream);

/* MXFP4 W4A16 on a weight in the MXFP4 decode layout: C = A . W^T, K % 128 == 0;
 * the decode GEMV for 1 <= M <= 16 (any such K), the prefill GEMM on the same
 * layout for larger M (mxfp4_gemm_w4a16's result, bit for bit).  Arithmetic and
 * tolerance as mxfp4_gemm_w4a16.  FP4_ERR_SHAPE for the same 2 GiB limits as
 * gemm_w4a16_decode, for any M, checked before anything is launched. */
fp4_status mxfp4_gemm_w4a16_decode(const void *a, int64_t M, int64_t K, int64_t lda, const uint8_t *w_codes_p,
                                   const uint8_t *w_scales_p, int64_t N, void *c, fp4_dtype ct, int64_t ldc,
                                   hipStream_t stream);

/* MXFP4 W4A4 GEMM on segment-major operands (eefocus.com edge-FP4 article, "FP4
 * as the next core standard": MXFP4, 32-element blocks with an E8M0 scale).  The
 * same product as mxfp4_gemm_w4a4, bit for bit, with W in the MXFP4 decode layout
 * (mxfp4_pack_decode) instead of row-major: a 256-row panel's 128-element K
 * segment is then contiguous, which is how the kernel reads it.  A (bf16
 * [M][lda]) is quantized with `rule` into `ws` in the same layout (codes
 * [K/128][M][64] at ws, E8M0 [K/128][M][4] at the next 256-byte boundary).
 * K % 128 == 0, M * K / 2 and N * K / 2 below 2^31 (FP4_ERR_SHAPE otherwise,
 * checked before A is quantized); FP4_ERR_WORKSPACE for a null, unaligned or short ws.  C [M][ldc] fp32 or bf16
 * is written; nothing is allocated. */
size_t mxfp4_gemm_w4a4_seg_workspace(int64_t M, int64_t K);
fp4_status mxfp4_gemm_w4a4_seg(const void *a, int64_t M, int64_t K, int64_t lda, fp4_mx_rule rule,
                               const uint8_t *w_codes_p, const uint8_t *w_scales_p, int64_t N, void *c,
                               fp4_dtype ct, int64_t ldc, void *ws, size_t ws_bytes, hipStream_t stream);

/* The GEMM half of mxfp4_gemm_w4a4_seg: A and W both MXFP4 in the segment-major
 * (decode) layout, codes [K/128][rows][64], scales [K/128][rows][4]. */
fp4_status mxfp4_gemm_prequant_seg(const uint8_t *a_codes_p, const uint8_t *a_scales_p, int64_t M, int64_t K,
                                   const uint8_t *w_codes_p, const uint8_t *w_scales_p, int64_t N, void *c,
                                   fp4_dtype ct, int64_t ldc, hipStream_t stream);

/* ---- W4A8: FP4 weights x FP8 activations (eefocus.com edge-FP4 article: an NPU
 * with native W4A8, weights quantized to FP4 and activations to FP8).  Both
 * operands take the OCP MX form: MXFP4 weights, MXFP8 activations. ---- */

/* MXFP8 quantize: x [rows][ldx] (fp32 or bf16) -> codes uint8 [rows][cols]
 * (E4M3FN, sign kept), scales uint8 [rows][cols/32] (E8M0).  Per 32-element
 * block: rule FP4_MX_OCP_FLOOR: 2^k with k = floor(log2 amax) - 8 (the block
 * maximum may saturate at 448); FP4_MX_CEIL: the smallest 2^k with 448 2^k >=
 * amax.  Elements: E4M3 round-to-nearest-even with saturation of |x| / 2^k; a
 * zero block gets scale byte 0.  cols % 32 == 0. */
fp4_status mxfp8_quantize(const void *x, fp4_dtype xt, int64_t rows, int64_t cols, int64_t ldx,
                          uint8_t *codes, uint8_t *scales, fp4_mx_rule rule, int32_t *nonfinite,
                          hipStream_t stream);

/* Workspace bytes mxfp4_gemm_w4a8 needs: A's MXFP8 codes | scales, each at a
 * 256-byte boundary. */
size_t mxfp4_gemm_w4a8_workspace(int64_t M, int64_t K);

/* W4A8 GEMM: the bf16 A is quantized to MXFP8 with `rule` into `ws`, then
 * C = A_q . W^T on gfx950's block-scaled matrix instruction with FP8 and FP4
 * operands (exact products, fp32 accumulation).  W MXFP4 [N][K].  K % 128 == 0,
 * M * K (A's MXFP8 bytes) and N * K / 2 below 2^31 (FP4_ERR_SHAPE otherwise,
 * checked before anything is launched).  Tolerance as the other GEMMs, against
 * fp64 over the dequantized operands. */
fp4_status mxfp4_gemm_w4a8(const void *a, int64_t M, int64_t K, int64_t lda, fp4_mx_rule rule,
                           const uint8_t *w_codes, const uint8_t *w_scales, int64_t N, void *c,
                           fp4_dtype ct, int64_t ldc, void *ws, size_t ws_bytes, hipStream_t stream);

/* The GEMM half of mxfp4_gemm_w4a8 on an already-quantized MXFP8 A (codes
 * [M][K], scales [M][K/32]). */
fp4_status mxfp4_gemm_w4a8_prequant(const uint8_t *a_codes, const uint8_t *a_scales, int64_t M, int64_t K,
                                    const uint8_t *w_codes, const uint8_t *w_scales, int64_t N, void *c,
                                    fp4_dtype ct, int64_t ldc, hipStream_t stream);

/* W4A8 with W in the MXFP4 decode layout (mxfp4_pack_decode: codes [K/128][N][64],
 * scales [K/128][N][4]); A as in mxfp4_gemm_w4a8.  The same result as
 * mxfp4_gemm_w4a8 / _prequant on the row-major W, bit for bit; the weight's
 * 128-element segments are then contiguous panels, which the kernel copies whole.
 * Arguments, workspace and errors as those two. */
fp4_status mxfp4_gemm_w4a8_seg(const void *a, int64_t M, int64_t K, int64_t lda, fp4_mx_rule rule,
                               const uint8_t *w_codes_p, const uint8_t *w_scales_p, int64_t N, void *c,
                               fp4_dtype ct, int64_t ldc, void *ws, size_t ws_bytes, hipStream_t stream);
fp4_status mxfp4_gemm_w4a8_prequant_seg(const uint8_t *a_codes, const uint8_t *a_scales, int64_t M, int64_t K,
                                        const uint8_t *w_codes_p, const uint8_t *w_scales_p, int64_t N, void *c,
                                        fp4_dtype ct, int64_t ldc, hipStream_t stream);

/* ---------------------------------------------------- grouped (MoE) ------ */

/* Grouped GEMMs for mixture-of-experts layers (eefocus.com edge-FP4 article, "FP4
 * as the next core standard": MoE expert weights stored as MXFP4; aixq.cc article
 * on Unsloth's Dynamic NVFP4, throughput section: a mixture-of-experts model run
 * with NVFP4 weights, and all-W4A4 in its "Fast" form).
 *
 * One weight per group (expert), stacked: codes [groups][N][K/2], scales
 * [groups][N][K/16] (NVFP4, E4M3) or [groups][N][K/32] (MXFP4, E8M0), NVFP4
 * tensor scales [groups] floats.  The `rows` grouped rows are the rows of C
 * [rows][ldc]; group e owns rows group_offs[e] .. group_offs[e+1]-1 and
 *   C[t] = A[row_index[t]] . W_e^T      (A[t] when row_index is null),
 * so a router's permutation is applied while A is loaded and C comes out in
 * grouped order.  A has a_rows rows; without row_index a_rows >= rows.
 *
 * group_offs (device, int32 [groups+1]) must be nondecreasing from 0 to rows,
 * and row_index (device, int32 [rows]) entries must lie in [0, a_rows).  Other
 * values give unspecified C but no access outside the buffers: offsets are
 * clamped to [0, rows], and a row index outside A reads as a zero row.  Empty
 * groups are allowed.  rows == 0 returns FP4_OK once groups, group_offs, K, N
 * and the output dtype check out, touching nothing (A, W, C may be null then).
 * groups <= 65536.
 * Errors (checked on the host, nothing launched): FP4_ERR_SHAPE for K not a
 * multiple of 64 (NVFP4) or 128 (MXFP4), A past 2 GiB (its bf16 rows, or for
 * W4A4 its packed codes), one group's weight codes past 2 GiB, or a tile grid of
 * 2^31 workgroups or more; FP4_ERR_NULL, FP4_ERR_LAYOUT as the other GEMMs.
 * nvfp4_grouped_gemm_w4a4 checks all of these before its quantizer runs.
 * Tolerance as the ungrouped GEMMs, row by row. */

/* NVFP4 weights, bf16 A [a_rows][lda]: each weight widened exactly to bf16,
 * fp32 accumulation, times the group's tensor scale. */
fp4_status nvfp4_grouped_gemm_w4a16(const void *a, int64_t a_rows, int64_t K, int64_t lda,
                                    const int32_t *row_index, const int32_t *group_offs, int64_t groups,
                                    int64_t rows, const uint8_t *w_codes, const uint8_t *w_scales,
                                    const float *w_tscale, int64_t N, void *c, fp4_dtype ct, int64_t ldc,
                                    hipStream_t stream);

/* MXFP4 weights, bf16 A: weights widened exactly (E2M1 times a power of two). */
fp4_status mxfp4_grouped_gemm_w4a16(const void *a, int64_t a_rows, int64_t K, int64_t lda,
                                    const int32_t *row_index, const int32_t *group_offs, int64_t groups,
                                    int64_t rows, const uint8_t *w_codes, const uint8_t *w_scales, int64_t N,
                                    void *c, fp4_dtype ct, int64_t ldc, hipStream_t stream);

/* Workspace bytes of nvfp4_grouped_gemm_w4a4: A's per-row NVFP4 form, laid out
 * as gemm_w4a4's per-row workspace for a_rows x K. */
size_t nvfp4_grouped_gemm_w4a4_workspace(int64_t a_rows, int64_t K);

/* NVFP4 W4A4: every A row (token) is quantized once, per row, into `ws`; the
 * grouped GEMM then reads the packed rows through row_index. */
fp4_status nvfp4_grouped_gemm_w4a4(const void *a, int64_t a_rows, int64_t K, int64_t lda,
                                   const int32_t *row_index, const int32_t *group_offs, int64_t groups,
                                   int64_t rows, const uint8_t *w_codes, const uint8_t *w_scales,
                                   const float *w_tscale, int64_t N, void *c, fp4_dtype ct, int64_t ldc, void *ws,
                                   size_t ws_bytes, hipStream_t stream);

/* The GEMM half of nvfp4_grouped_gemm_w4a4 on a per-row NVFP4 A (codes
 * [a_rows][K/2], scales [a_rows][K/16], a_tscale [a_rows]). */
fp4_status nvfp4_grouped_gemm_w4a4_prequant(const uint8_t *a_codes, const uint8_t *a_scales,
                                            const float *a_tscale, int64_t a_rows, int64_t K,
                                            const int32_t *row_index, const int32_t *group_offs,
                                            int64_t groups, int64_t rows, const uint8_t *w_codes,
                                            const uint8_t *w_scales, const float *w_tscale, int64_t N,
                                            void *c, fp4_dtype ct, int64_t ldc, hipStream_t stream);

/* ---------------------------------------------------------- measurement --
 * fp4blk_read_ceiling: reads `bytes` bytes at `buf` once, with `grid`
 * workgroups of 512 threads striding over 16-byte words, and computes nothing
 * from them.  Its duration is the reference for the decode GEMV, which streams
 * its weight exactly once per call and is therefore bound by memory bandwidth
 * (edge-FP4 article, eefocus.com, section on the trade-offs of compute, memory
 * and precision).  A measurement aid, not part of the quantization path.
 * buf: device, 16-byte aligned; bytes: > 0, a multiple of 16; grid: 1..65535;
 * sink: device uint32, written only in the (practically never taken) case that
 * the XOR of all words equals a fixed constant.  FP4_ERR_NULL / _SHAPE /
 * _LAYOUT on bad arguments, nothing launched. */
fp4_status fp4blk_read_ceiling(const void *buf, size_t bytes, int grid, uint32_t *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FP4BLK_H */
