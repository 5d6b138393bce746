/*
 * fp4_oracle.c -- plain, slow, obviously-correct CPU oracle for block-scaled
 * 4-bit quantization (NVFP4, MXFP4) and the GEMMs it feeds.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or constant with the HIP library; the two meet only through the seeded
 * inputs they are both given.
 *
 * Sources (the pages are cited by title and section):
 *  - "NVFP4" (newton.com.tw wiki), section "Technical principle" (技術原理):
 *    E2M1 elements (1 sign, 2 exponent, 1 mantissa bit, range about -6..6);
 *    16-value micro-blocks each sharing an E4M3 FP8 scale that may be a
 *    non-power-of-two; one FP32 scale for the whole tensor; about 4.5 bits per
 *    value.
 *  - Edge-FP4 article (eefocus.com, "英伟达、AMD、安谋科技集体押注…"), section
 *    "FP4 as the next core standard" (FP4被视为下一代AI计算的核心标准): OCP MX
 *    block floating point, 32-element blocks sharing one E8M0 scale, E2M1
 *    elements, 4.25 bits per weight.
 *  - Unsloth Dynamic NVFP4 article (aixq.cc), section "Core difference: W4A4 vs
 *    W4A16": W4A16 dequantizes 4-bit weights to 16 bits before a 16-bit matmul;
 *    W4A4 quantizes the activations too.
 *
 * Readings where the pages leave a step open (each listed in the design notes):
 *  - E4M3 is the OCP E4M3FN variant: bias 7, no infinities, 0x7F/0xFF NaN,
 *    largest finite 448.
 *  - tensor scale s = fl32(amax / 2688), 2688 = 6 * 448, stored as is;
 *    block scale byte = E4M3 round-to-nearest-even with saturation of
 *    fl32(block_amax / fl32(6 * s)); element code = E2M1 round-to-nearest-even
 *    with saturation of fl32(x / fl32(E4M3(byte) * s)).  Division, not a
 *    multiply by a reciprocal.
 *  - E2M1 ties go to the even mantissa bit; the sign of zero is kept.
 *  - a zero block gets byte 0x00; if the block divisor is zero every code in
 *    the block is a signed zero.
 *  - MXFP4 scale exponent: OCP rule k = floor(log2 block_amax) - 2, or the
 *    "ceil" rule (smallest k with 6 * 2^k >= block_amax); k clamped to
 *    [-127, 127]; a zero block gets byte 0.
 *  - codes: low nibble holds the even column; scales row-major [rows][cols/block].
 *
 * All fp32 arithmetic below is IEEE single precision, round to nearest even,
 * with no contraction and no flush-to-zero (built with -ffp-contract=off, no
 * fast-math).  fp64 is used only where the result is exact.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define FP4O_F32 0
#define FP4O_BF16 1

/* ---------------------------------------------------------------- codecs -- */

/* E2M1 code -> value.  Bit fields s|e e|m; e == 0 is the subnormal 0.5*m,
 * otherwise 2^(e-1) * (1 + m/2).  ("NVFP4", Technical principle: E2M1.) */
double fp4o_e2m1_decode(uint8_t c)
{
    int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* value -> E2M1 code: nearest grid point of {0,0.5,1,1.5,2,3,4,6}, ties to the
 * even mantissa bit, magnitudes above 6 saturate to 6.  The decision points are
 * the midpoints between neighbours; at a midpoint the neighbour with m == 0
 * wins (0, 1, 2, 4 are even; 0.5, 1.5, 3, 6 are odd). */
uint8_t fp4o_e2m1_encode(double v)
{
    double a = fabs(v);
    uint8_t m;
    if (a <= 0.25)      m = 0;   /* midpoint 0|0.5   -> 0   (even) */
    else if (a < 0.75)  m = 1;   /* midpoint 0.5|1   -> 1   (even) */
    else if (a <= 1.25) m = 2;   /* midpoint 1|1.5   -> 1   (even) */
    else if (a < 1.75)  m = 3;   /* midpoint 1.5|2   -> 2   (even) */
    else if (a <= 2.5)  m = 4;   /* midpoint 2|3     -> 2   (even) */
    else if (a < 3.5)   m = 5;   /* midpoint 3|4     -> 4   (even) */
    else if (a <= 5.0)  m = 6;   /* midpoint 4|6     -> 4   (even) */
    else                m = 7;   /* saturate at 6 (also +inf; NaN is a precondition) */
    return (uint8_t)((signbit(v) ? 8 : 0) | m);
}

/* E4M3FN byte -> value: s|eeee|mmm, bias 7; e == 0 is subnormal m * 2^-9;
 * 0x7F / 0xFF are NaN; no infinities. */
double fp4o_e4m3_decode(uint8_t b)
{
    int s = (b >> 7) & 1, e = (b >> 3) & 15, m = b & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) mag = ldexp((double)m, -9);
    else        mag = ldexp(8.0 + m, e - 10);  /* (1 + m/8) * 2^(e-7) */
    return s ? -mag : mag;
}

/* non-negative fp32 -> E4M3FN byte, round to nearest even, saturating at 448
 * (0x7E).  +inf saturates; NaN (a precondition violation) maps to 0x7F. */
uint8_t fp4o_e4m3_encode_sat(float qf)
{
    double q = (double)qf;
    if (isnan(q)) return 0x7F;
    if (q >= 448.0) return 0x7E;
    if (q < 0x1p-6) {
        /* subnormal: m * 2^-9, m = RNE(q * 2^9) in 0..8; m == 8 is 0x08 = 2^-6 */
        return (uint8_t)nearbyint(q * 512.0);
    }
    int e;
    double fr = frexp(q, &e);          /* q = fr * 2^e, fr in [0.5, 1) */
    int E = e - 1;                     /* q = (2 fr) * 2^E */
    double m = nearbyint((2.0 * fr - 1.0) * 8.0);
    if (m == 8.0) { m = 0.0; E += 1; }
    int biased = E + 7;
    if (biased > 15 || (biased == 15 && m > 6.0)) return 0x7E;
    return (uint8_t)((biased << 3) | (int)m);
}

/* E8M0 byte -> 2^(b-127); 0xFF is NaN.  (Edge-FP4 article, OCP MX section.) */
double fp4o_e8m0_decode(uint8_t b)
{
    if (b == 0xFF) return NAN;
    return ldexp(1.0, (int)b - 127);
}

/* fp32 -> bfloat16 bits, round to nearest even (NaN kept quiet). */
uint16_t fp4o_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu))
        return (uint16_t)((u >> 16) | 0x40);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

static float bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static float load_x(const void *x, int dtype, int64_t i)
{
    return dtype == FP4O_F32 ? ((const float *)x)[i] : bf16_to_f32(((const uint16_t *)x)[i]);
}

/* bulk codec entry points for the tests */
void fp4o_e2m1_encode_f32(const float *v, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = fp4o_e2m1_encode((double)v[i]);
}

void fp4o_e4m3_encode_f32(const float *v, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = fp4o_e4m3_encode_sat(v[i]);
}

void fp4o_f32_to_bf16_n(const float *v, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = fp4o_f32_to_bf16(v[i]);
}

/* ------------------------------------------------------------- NVFP4 ------ */

/* amax = max |x| over rows r0..r1 (fp32 compare; bf16 widened exactly). */
static float amax_rows(const void *x, int dtype, int64_t r0, int64_t r1, int64_t cols, int64_t ldx)
{
    float amax = 0.0f;
    for (int64_t r = r0; r < r1; ++r)
        for (int64_t k = 0; k < cols; ++k) {
            float a = fabsf(load_x(x, dtype, r * ldx + k));
            if (a > amax) amax = a;
        }
    return amax;
}

/* Quantize one row with tensor scale s (the "NVFP4" page's two-level scheme). */
static void nvfp4_quantize_row(const void *x, int dtype, int64_t r, int64_t cols, int64_t ldx,
                               float s, uint8_t *codes, uint8_t *scales)
{
    const float six_s = 6.0f * s;
    for (int64_t j = 0; j < cols / 16; ++j) {
        float xv[16];
        float amax_b = 0.0f;
        for (int i = 0; i < 16; ++i) {
            xv[i] = load_x(x, dtype, r * ldx + j * 16 + i);
            float a = fabsf(xv[i]);
            if (a > amax_b) amax_b = a;
        }
        uint8_t b = (amax_b == 0.0f) ? 0x00 : fp4o_e4m3_encode_sat(amax_b / six_s);
        scales[r * (cols / 16) + j] = b;
        float d = (float)fp4o_e4m3_decode(b) * s;
        for (int i = 0; i < 16; i += 2) {
            uint8_t c0, c1;
            if (d == 0.0f) {
                c0 = signbit(xv[i]) ? 8 : 0;
                c1 = signbit(xv[i + 1]) ? 8 : 0;
            } else {
                float q0 = xv[i] / d, q1 = xv[i + 1] / d;
                c0 = fp4o_e2m1_encode((double)q0);
                c1 = fp4o_e2m1_encode((double)q1);
            }
            codes[r * (cols / 2) + (j * 16 + i) / 2] = (uint8_t)(c0 | (c1 << 4));
        }
    }
}

/* NVFP4 quantize.  per_row == 0: one tensor scale (tscale[0]) from the whole
 * tensor's amax; per_row == 1: each row is its own tensor (tscale[rows]).
 * cols must be a multiple of 16 (checked by the caller).  Returns 0. */
int fp4o_nvfp4_quantize(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                        uint8_t *codes, uint8_t *scales, float *tscale, int per_row)
{
    if (!per_row) {
        float amax = 0.0f;
#pragma omp parallel for reduction(max : amax) schedule(static)
        for (int64_t r = 0; r < rows; ++r) {
            float a = amax_rows(x, dtype, r, r + 1, cols, ldx);
            if (a > amax) amax = a;
        }
        float s = amax / 2688.0f;
        tscale[0] = s;
#pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < rows; ++r)
            nvfp4_quantize_row(x, dtype, r, cols, ldx, s, codes, scales);
    } else {
#pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < rows; ++r) {
            float s = amax_rows(x, dtype, r, r + 1, cols, ldx) / 2688.0f;
            tscale[r] = s;
            nvfp4_quantize_row(x, dtype, r, cols, ldx, s, codes, scales);
        }
    }
    return 0;
}

/* NVFP4 dequantize to fp32: y = fl32(fl32(E2M1(c) * E4M3(b)) * s).  The inner
 * product has at most 6 significant bits, so it is exact in fp32 and the only
 * rounding is the multiply by s. */
void fp4o_nvfp4_dequantize(const uint8_t *codes, const uint8_t *scales, const float *tscale,
                           int per_row, int64_t rows, int64_t cols, float *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        float s = per_row ? tscale[r] : tscale[0];
        for (int64_t k = 0; k < cols; ++k) {
            uint8_t byte = codes[r * (cols / 2) + k / 2];
            uint8_t c = (k & 1) ? (byte >> 4) : (byte & 15);
            float p = (float)(fp4o_e2m1_decode(c) * fp4o_e4m3_decode(scales[r * (cols / 16) + k / 16]));
            y[r * cols + k] = p * s;
        }
    }
}

/* NVFP4 operand as exact reals in fp64: E2M1(c) * E4M3(b) * s (at most 6 + 24
 * significant bits, so exact).  This is what a GEMM contracts over. */
void fp4o_nvfp4_to_f64(const uint8_t *codes, const uint8_t *scales, const float *tscale,
                       int per_row, int64_t rows, int64_t cols, double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double s = per_row ? tscale[r] : tscale[0];
        for (int64_t k = 0; k < cols; ++k) {
            uint8_t byte = codes[r * (cols / 2) + k / 2];
            uint8_t c = (k & 1) ? (byte >> 4) : (byte & 15);
            y[r * cols + k] = fp4o_e2m1_decode(c) * fp4o_e4m3_decode(scales[r * (cols / 16) + k / 16]) * s;
        }
    }
}

/* ------------------------------------------------------------- MXFP4 ------ */

/* MXFP4 quantize (OCP MX, 32-element blocks, E8M0 scale, no tensor scale).
 * rule 0: k = floor(log2 amax_b) - 2 (E2M1's largest exponent is 2);
 * rule 1: the smallest k with 6 * 2^k >= amax_b.
 * k is clamped to [-127, 127], byte = k + 127; each element is x * 2^-k
 * (exact) rounded to E2M1 with saturation. */
void fp4o_mxfp4_quantize(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                         uint8_t *codes, uint8_t *scales, int rule)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t j = 0; j < cols / 32; ++j) {
            float xv[32];
            float amax_b = 0.0f;
            for (int i = 0; i < 32; ++i) {
                xv[i] = load_x(x, dtype, r * ldx + j * 32 + i);
                float a = fabsf(xv[i]);
                if (a > amax_b) amax_b = a;
            }
            int k = 0;
            uint8_t byte = 0;
            int zero = (amax_b == 0.0f);
            if (!zero) {
                int e;
                (void)frexp((double)amax_b, &e);
                int E = e - 1;                         /* floor(log2 amax_b), exact */
                if (rule == 0) k = E - 2;
                else k = ((double)amax_b <= ldexp(1.5, E)) ? E - 2 : E - 1;
                if (k < -127) k = -127;
                if (k > 127) k = 127;
                byte = (uint8_t)(k + 127);
            }
            scales[r * (cols / 32) + j] = byte;
            for (int i = 0; i < 32; i += 2) {
                uint8_t c0, c1;
                if (zero) {
                    c0 = signbit(xv[i]) ? 8 : 0;
                    c1 = signbit(xv[i + 1]) ? 8 : 0;
                } else {
                    c0 = fp4o_e2m1_encode(ldexp((double)xv[i], -k));
                    c1 = fp4o_e2m1_encode(ldexp((double)xv[i + 1], -k));
                }
                codes[r * (cols / 2) + (j * 32 + i) / 2] = (uint8_t)(c0 | (c1 << 4));
            }
        }
    }
}

/* MXFP4 dequantize to fp32: E2M1(c) * 2^(byte-127), exact whenever it is in
 * fp32's range. */
void fp4o_mxfp4_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t rows,
                           int64_t cols, float *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < cols; ++k) {
            uint8_t byte = codes[r * (cols / 2) + k / 2];
            uint8_t c = (k & 1) ? (byte >> 4) : (byte & 15);
            y[r * cols + k] = (float)(fp4o_e2m1_decode(c) * fp4o_e8m0_decode(scales[r * (cols / 32) + k / 32]));
        }
}

void fp4o_mxfp4_to_f64(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols,
                       double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < cols; ++k) {
            uint8_t byte = codes[r * (cols / 2) + k / 2];
            uint8_t c = (k & 1) ? (byte >> 4) : (byte & 15);
            y[r * cols + k] = fp4o_e2m1_decode(c) * fp4o_e8m0_decode(scales[r * (cols / 32) + k / 32]);
        }
}

/* MXFP8 quantize (the FP8 activations of W4A8; edge-FP4 article, section on
 * W4A8 in the NPU paragraph: weights FP4, activations FP8).  Reading: OCP MX
 * blocks of 32 elements with an E8M0 scale, E4M3FN elements.
 * rule 0: k = floor(log2 amax_b) - 8 (E4M3's largest exponent is 8);
 * rule 1: the smallest k with 448 * 2^k >= amax_b.
 * k is clamped to [-127, 127], byte = k + 127; each element is |x| * 2^-k
 * (exact) rounded to E4M3 with saturation at 448, sign kept (a negative value
 * that rounds to 0 is 0x80).  A zero block gets byte 0 and signed zeros. */
void fp4o_mxfp8_quantize(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                         uint8_t *codes, uint8_t *scales, int rule)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t j = 0; j < cols / 32; ++j) {
            float xv[32];
            float amax_b = 0.0f;
            for (int i = 0; i < 32; ++i) {
                xv[i] = load_x(x, dtype, r * ldx + j * 32 + i);
                float a = fabsf(xv[i]);
                if (a > amax_b) amax_b = a;
            }
            int k = 0;
            uint8_t byte = 0;
            int zero = (amax_b == 0.0f);
            if (!zero) {
                int e;
                (void)frexp((double)amax_b, &e);
                int E = e - 1;                         /* floor(log2 amax_b), exact */
                if (rule == 0) k = E - 8;
                else k = ((double)amax_b <= ldexp(1.75, E)) ? E - 8 : E - 7;
                if (k < -127) k = -127;
                if (k > 127) k = 127;
                byte = (uint8_t)(k + 127);
            }
            scales[r * (cols / 32) + j] = byte;
            for (int i = 0; i < 32; ++i) {
                uint8_t sign = signbit(xv[i]) ? 0x80 : 0x00;
                uint8_t mag = zero ? 0 : fp4o_e4m3_encode_sat((float)ldexp(fabs((double)xv[i]), -k));
                codes[r * cols + j * 32 + i] = (uint8_t)(sign | mag);
            }
        }
    }
}

/* MXFP8 dequantize to fp64: E4M3(c) * 2^(byte-127), exact. */
void fp4o_mxfp8_to_f64(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols,
                       double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < cols; ++k)
            y[r * cols + k] = fp4o_e4m3_decode(codes[r * cols + k]) * fp4o_e8m0_decode(scales[r * (cols / 32) + k / 32]);
}

/* ------------------------------------------------------------- INT4 ------- */

/* INT4 linear quantization, the integer baseline FP4 is compared with (edge-FP4
 * article, section on why FP4 suits compression: INT4's evenly spaced levels
 * lack a floating-point dynamic range; NVFP4 wiki, competition section: INT4
 * versions lose more accuracy than FP4 on some tasks).  The pages fix no INT4
 * layout; this one is symmetric: levels -7..7, one step d per block of `block`
 * elements along a row, element = round-half-even(x / d) saturated at +-7.  The
 * step d comes from the block's amax_b in one of four containers:
 *   kind 0: d = fl32(amax_b / 7)                        (fp32 per block)
 *   kind 1: d = bf16_rne(fl32(amax_b / 7))               (bf16 per block)
 *   kind 2: d = E4M3(b) * s, s = fl32(amax_tensor / (448 * 7)),
 *           b = E4M3_rne_sat(fl32(amax_b / fl32(7 s)))   (NVFP4's container)
 *   kind 3: d = 2^k, the smallest k with 7 * 2^k >= amax_b (MXFP4's container)
 * A zero block has d = 0 and codes 0.  codes [rows][cols] int8; dstep
 * [rows][cols / block] the decoded steps; *tensor_scale gets s (kind 2). */
void fp4o_int4_quantize(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ldx, int block,
                        int kind, int8_t *codes, double *dstep, float *tensor_scale)
{
    float s = 0.0f;
    if (kind == 2) {
        float amax = 0.0f;
        for (int64_t r = 0; r < rows; ++r) {
            float a = amax_rows(x, dtype, r, r + 1, cols, ldx);
            if (a > amax) amax = a;
        }
        s = amax / (448.0f * 7.0f);
        if (tensor_scale) *tensor_scale = s;
    }
    const int64_t nb = cols / block;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t j = 0; j < nb; ++j) {
            float amax_b = 0.0f;
            for (int i = 0; i < block; ++i) {
                float a = fabsf(load_x(x, dtype, r * ldx + j * block + i));
                if (a > amax_b) amax_b = a;
            }
            double d = 0.0;
            if (amax_b > 0.0f) {
                if (kind == 0) {
                    d = (double)(amax_b / 7.0f);
                } else if (kind == 1) {
                    d = (double)bf16_to_f32(fp4o_f32_to_bf16(amax_b / 7.0f));
                } else if (kind == 2) {
                    d = fp4o_e4m3_decode(fp4o_e4m3_encode_sat(amax_b / (7.0f * s))) * (double)s;
                } else {
                    int e;
                    (void)frexp((double)amax_b / 7.0, &e);   /* amax/7 in [2^(e-1), 2^e) */
                    int k = e;
                    if (ldexp(7.0, k - 1) >= (double)amax_b) k -= 1;   /* exact power-of-two case */
                    d = ldexp(1.0, k);
                }
            }
            dstep[r * nb + j] = d;
            for (int i = 0; i < block; ++i) {
                int8_t q = 0;
                if (d > 0.0) {
                    double v = nearbyint((double)load_x(x, dtype, r * ldx + j * block + i) / d);
                    if (v > 7.0) v = 7.0;
                    if (v < -7.0) v = -7.0;
                    q = (int8_t)v;
                }
                codes[r * cols + j * block + i] = q;
            }
        }
    }
}

/* -------------------------------------------------------------- GEMM ------ */

/* C[m][n] = sum_k a[m][k] * w[n][k] in fp64, and T[m][n] = sum_k |a w|
 * (the tolerance scale).  A plain triple loop over exact operands. */
void fp4o_gemm_f64(const double *a, const double *w, int64_t M, int64_t N, int64_t K,
                   double *c, double *t)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, abs_acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = a[m * K + k] * w[n * K + k];
                acc += p;
                abs_acc += fabs(p);
            }
            c[m * N + n] = acc;
            if (t) t[m * N + n] = abs_acc;
        }
}

/* threads an OpenMP region of this library uses (for reporting the CPU baseline) */
#ifdef _OPENMP
#include <omp.h>
int fp4o_num_threads(void) { return omp_get_max_threads(); }
#else
int fp4o_num_threads(void) { return 1; }
#endif
