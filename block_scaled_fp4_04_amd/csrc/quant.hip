// quant.hip -- NVFP4 and MXFP4 quantize / dequantize kernels for gfx950.
//
// NVFP4 ("NVFP4", newton.com.tw wiki, section "Technical principle"): a tensor
// is cut into 16-value micro-blocks along its rows; each block gets one E4M3
// scale byte and the tensor one FP32 scale; elements are E2M1.
// MXFP4 (edge-FP4 article, eefocus.com, section "FP4 as the next core
// standard"): 32-element blocks, one E8M0 byte each, E2M1 elements.
//
// Work unit: one lane owns 8 consecutive elements of a row (one or two 16-byte
// loads), so a wave reads 512 contiguous elements per instruction pair and
// writes its 8 codes as one 32-bit store.  A 16-block is a lane pair, a
// 32-block a lane quad; block maxima are exchanged with DPP quad permutes.
//
// All fp32 arithmetic here is IEEE round-to-nearest-even: the library is built
// with correctly rounded fp32 division, no contraction, denormals kept.
#include "device_common.h"
#include "internal.h"

#pragma clang fp contract(off)

namespace fp4k {

template <typename T>
struct Vec8;

template <>
struct Vec8<float> {
    static __device__ __forceinline__ void load(const float *p, float v[8])
    {
        const float4 a = *reinterpret_cast<const float4 *>(p);
        const float4 b = *reinterpret_cast<const float4 *>(p + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
};

template <>
struct Vec8<uint16_t> {
    static __device__ __forceinline__ void load(const uint16_t *p, float v[8])
    {
        const uint4 a = *reinterpret_cast<const uint4 *>(p);
        const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    }
};

__device__ __forceinline__ float amax8(const float v[8], int &bad)
{
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float a = __builtin_fabsf(v[i]);
        bad |= !__builtin_isfinite(a);
        m = fmaxf(m, a);
    }
    return m;
}

// Streaming (non-temporal) stores for the quantizers' outputs: each byte is written
// once and read, if at all, by a later kernel, so it need not stay in the caches.
// (The dequantizers keep ordinary stores: theirs cover 16 bytes of every 32 or 64
// per instruction, and as streaming stores those ran at half the rate.)
__device__ __forceinline__ void st_nt8(uint32_t v, uint8_t *p) { __builtin_nontemporal_store((uint8_t)v, p); }
__device__ __forceinline__ void st_nt32(uint32_t v, uint8_t *p)
{
    __builtin_nontemporal_store(v, reinterpret_cast<uint32_t *>(p));
}
__device__ __forceinline__ void st_nt64(uint32_t lo, uint32_t hi, uint8_t *p)
{
    __builtin_nontemporal_store(u32x2{lo, hi}, reinterpret_cast<u32x2 *>(p));
}

// ------------------------------------------- division by a shared divisor --
//
// Every value of a 16-block is divided by the same step d = fl32(E4M3(b) s), and
// every block byte of a row or tensor by the same 6 s.  gfx950's correctly
// rounded fp32 division (as the compiler emits it for a / b) is: pre-scale both
// operands (div_scale), y = rcp(b) refined by one Newton step, q0 = a y, then two
// remainder corrections q <- q + (a - b q) y by FMA, and a final special-value
// fix-up (div_fixup).  Only the product and the corrections depend on a, so
// rcp_refined() computes y once per divisor and div_refined() repeats the rest
// per value: a product and four FMAs in place of about eleven instructions.
// The pre-scaling is the identity (and the fix-up returns its input) when b and
// 1/b are normal, a is zero or not tiny (|a| >= 2^-103) and a / b is neither
// denormal nor within 2^96 of overflow.  nv_fast_scale(s) admits tensor scales
// s in [2^-50, 2^50]; every divisor is then in [2^-59, 2^59], and every quotient
// that can decide an E2M1 code or an E4M3 byte (a / b >= 2^-11) has a normal
// numerator, so it is formed exactly as by the division.  Smaller quotients
// land on code 0 / byte 0 either way.  Other scales take the IEEE division.

__device__ __forceinline__ bool nv_fast_scale(float s) { return s >= 0x1p-50f && s <= 0x1p50f; }

__device__ __forceinline__ float rcp_refined(float b)
{
    const float y0 = __builtin_amdgcn_rcpf(b);
    return __builtin_fmaf(__builtin_fmaf(-b, y0, 1.0f), y0, y0);
}

// Each correction is written q - (b q - a) y: the same value as q + (a - b q) y
// (round to nearest is symmetric, so the remainder is only negated), but a
// numerator of -0 then gives -0 (the sum -0 + -0), where the other order gives +0;
// so the quotient carries the sign of a in every case, as the division does.
__device__ __forceinline__ float div_refined(float a, float b, float y)
{
    const float q0 = a * y;
    const float q1 = __builtin_fmaf(-__builtin_fmaf(b, q0, -a), y, q0);
    return __builtin_fmaf(-__builtin_fmaf(b, q1, -a), y, q1);
}

// E4M3FN byte of one non-negative value (round to nearest even, saturating at 448).
__device__ __forceinline__ uint32_t e4m3_code_sat1(float q)
{
    typedef short v2i16 __attribute__((ext_vector_type(2)));
    const v2i16 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v2i16{0, 0}, fminf(q, 448.0f), 0.0f, 1.0f, false);
    return (uint32_t)(uint16_t)r[0] & 0xFFu;
}

// The E4M3 block byte and the codes of one 8-element unit (lanes 2i, 2i + 1 hold
// one 16-block) on the fast path: bm8 = max|v| over the unit, y6 = rcp_refined(6 s).
// A block whose byte is 0 divides by s 2^20 instead of 0: its quotients are then
// below 2^-27 and every code is the sign alone, as the definition asks.
__device__ __forceinline__ uint32_t nvfp4_unit_fast(const float v[8], float bm8, float s, float six_s, float y6,
                                                    uint32_t &code_word)
{
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const float bm = fmaxf(bm8, xor1(bm8));
    const uint32_t b = e4m3_code_sat1(div_refined(bm, six_s, y6));
    const f32x2 bv = __builtin_amdgcn_cvt_pk_f32_fp8((int)b, false);
    const float d = b ? bv[0] * s : s * 0x1p20f;
    const float y = rcp_refined(d);
    float q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = div_refined(v[i], d, y);
    code_word = e2m1x8_code(q);
    return b;
}

// Codes of 8 values under divisor d (d == 0: signed zeros), nibble i = value i.
__device__ __forceinline__ uint32_t nvfp4_codes8(const float v[8], float d)
{
    if (d == 0.0f) {
        uint32_t w = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) w |= ((__float_as_uint(v[i]) >> 28) & 8u) << (4 * i);
        return w;
    }
    float q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = v[i] / d;  // correctly rounded
    return e2m1x8_code(q);
}

// ------------------------------------------------------------------ amax --

// Per-block maxima of |x| over the whole tensor; partial[blockIdx.x].
template <typename T>
__global__ __launch_bounds__(256) void k_amax_partial(const T *__restrict__ x, uint32_t units,
                                                      FastDiv cv, int64_t ldx,
                                                      float *__restrict__ partial,
                                                      int32_t *__restrict__ nonfinite)
{
    float m = 0.0f;
    int bad = 0;
    for (uint32_t u = blockIdx.x * 256u + threadIdx.x; u < units; u += gridDim.x * 256u) {
        const uint32_t r = fdiv(u, cv);
        const uint32_t c8 = u - r * cv.d;
        float v[8];
        Vec8<T>::load(x + (int64_t)r * ldx + (int64_t)c8 * 8, v);
        m = fmaxf(m, amax8(v, bad));
    }
    m = wave_max(m);
    __shared__ float red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    if (bad && nonfinite) *nonfinite = 1;
    __syncthreads();
    if (threadIdx.x == 0) partial[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// tscale[0] = fl32(max(partial) / 2688).
__global__ __launch_bounds__(256) void k_tscale_finalize(const float *__restrict__ partial, int n,
                                                         float *__restrict__ tscale)
{
    float m = 0.0f;
    for (int i = threadIdx.x; i < n; i += 256) m = fmaxf(m, partial[i]);
    m = wave_max(m);
    __shared__ float red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) tscale[0] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])) / 2688.0f;
}

// --------------------------------------------------------- NVFP4 quantize --

// One 8-element unit under tensor scale s: lanes (2i, 2i+1) hold one 16-block.
__device__ __forceinline__ void nvfp4_unit(const float v[8], float s, float six_s,
                                           uint32_t *code_word, uint8_t *scale_byte, bool even)
{
    int dummy = 0;
    float bm = amax8(v, dummy);
    bm = fmaxf(bm, xor1(bm));
    const uint32_t b = bm == 0.0f ? 0u : e4m3x4_code_sat(bm / six_s, 0.0f, 0.0f, 0.0f) & 0xFFu;
    const float d = e4m3_value(b) * s;
    *code_word = nvfp4_codes8(v, d);
    if (even) *scale_byte = (uint8_t)b;
}

// Per-tensor mode: tensor scale read from device memory (written by
// k_tscale_finalize on the same stream).
template <typename T>
__global__ __launch_bounds__(256) void k_nvfp4_quant_tensor(const T *__restrict__ x, uint32_t units,
                                                            FastDiv cv, int64_t ldx, int64_t cols,
                                                            const float *__restrict__ tscale,
                                                            uint8_t *__restrict__ codes,
                                                            uint8_t *__restrict__ scales)
{
    const float s = tscale[0];
    const float six_s = 6.0f * s;
    const bool fast = nv_fast_scale(s);
    const float y6 = rcp_refined(six_s);
    for (uint32_t u = blockIdx.x * 256u + threadIdx.x; u < units; u += gridDim.x * 256u) {
        const uint32_t r = fdiv(u, cv);
        const uint32_t c8 = u - r * cv.d;
        float v[8];
        Vec8<T>::load(x + (int64_t)r * ldx + (int64_t)c8 * 8, v);
        uint32_t w;
        uint8_t *sp = scales + (int64_t)r * (cols / 16) + (c8 >> 1);
        if (fast) {
            int dummy = 0;
            const uint32_t b = nvfp4_unit_fast(v, amax8(v, dummy), s, six_s, y6, w);
            if ((c8 & 1u) == 0u) st_nt8(b, sp);
        } else {
            nvfp4_unit(v, s, six_s, &w, sp, (c8 & 1u) == 0u);
        }
        st_nt32(w, codes + (int64_t)r * (cols / 2) + (int64_t)c8 * 4);
    }
}

// Per-row mode: one workgroup per row; pass 1 finds the row amax, pass 2
// re-reads the row (from cache) and quantizes it.
template <typename T>
__global__ __launch_bounds__(256) void k_nvfp4_quant_rows(const T *__restrict__ x, int64_t rows,
                                                          int64_t cols, int64_t ldx,
                                                          uint8_t *__restrict__ codes,
                                                          uint8_t *__restrict__ scales,
                                                          float *__restrict__ tscale,
                                                          int32_t *__restrict__ nonfinite)
{
    __shared__ float red[4];
    const int64_t units = cols / 8;
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const T *xr = x + r * ldx;
        float m = 0.0f;
        int bad = 0;
        for (int64_t u = threadIdx.x; u < units; u += 256) {
            float v[8];
            Vec8<T>::load(xr + u * 8, v);
            m = fmaxf(m, amax8(v, bad));
        }
        if (bad && nonfinite) *nonfinite = 1;
        m = wave_max(m);
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
        __syncthreads();
        const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        __syncthreads();
        const float s = amax / 2688.0f;
        const float six_s = 6.0f * s;
        if (threadIdx.x == 0) tscale[r] = s;
        for (int64_t u = threadIdx.x; u < units; u += 256) {
            float v[8];
            Vec8<T>::load(xr + u * 8, v);
            uint32_t w;
            nvfp4_unit(v, s, six_s, &w, scales + r * (cols / 16) + (u >> 1), (u & 1) == 0);
            *reinterpret_cast<uint32_t *>(codes + r * (cols / 2) + u * 4) = w;
        }
    }
}

// Per-row mode for rows of at most 1024 U elements: one wave per row, four rows
// per workgroup.  Lane l owns the 16-blocks l, l + 64, ..., l + 64 (U - 1) of its
// row, so each block's byte, step and reciprocal are formed once, by one lane.
// All loads of the row go out at once (a buffer descriptor over the row returns
// zeros past its end), the row maximum is a wave reduction, and the row is
// quantized from registers: it is read from memory once and no barrier is
// needed.  bf16 rows keep their packed bits (maxima on the 16-bit magnitudes,
// which order like the values; 0x7F80 and above is Inf or NaN).
template <typename T, int U>
__global__ __launch_bounds__(256) void k_nvfp4_quant_rows_w(const T *__restrict__ x, int64_t rows, int cols,
                                                            int64_t ldx, uint8_t *__restrict__ codes,
                                                            uint8_t *__restrict__ scales, float *__restrict__ tscale,
                                                            int32_t *__restrict__ nonfinite)
{
    constexpr bool BF = sizeof(T) == 2;
    constexpr int LPB = BF ? 2 : 4;  // 16-byte loads per block
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (r >= rows) return;  // whole waves
    const int blocks = cols >> 4;
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<T *>(x + r * ldx), (short)0, cols * (int)sizeof(T), 0x00020000);
    u32x4 raw[U][LPB];
#pragma unroll
    for (int i = 0; i < U; ++i)
#pragma unroll
        for (int h = 0; h < LPB; ++h)
            raw[i][h] = __builtin_amdgcn_raw_buffer_load_b128(rx, (lane + 64 * i) * 16 * LPB + 16 * h, 0, 0);

    float bmax[U];  // max |v| of each block
    float m = 0.0f;
    int bad = 0;
#pragma unroll
    for (int i = 0; i < U; ++i) {
        if constexpr (BF) {
            typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
            u16x2 h[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint32_t mag = raw[i][k >> 2][k & 3] & 0x7FFF7FFFu;
                __builtin_memcpy(&h[k], &mag, 4);
            }
            const u16x2 t = __builtin_elementwise_max(
                __builtin_elementwise_max(__builtin_elementwise_max(h[0], h[1]), __builtin_elementwise_max(h[2], h[3])),
                __builtin_elementwise_max(__builtin_elementwise_max(h[4], h[5]), __builtin_elementwise_max(h[6], h[7])));
            const uint32_t mb = t[0] > t[1] ? t[0] : t[1];
            bad |= mb >= 0x7F80u;
            bmax[i] = __uint_as_float(mb << 16);
        } else {
            float a = 0.0f;
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const float v = __builtin_fabsf(__uint_as_float(raw[i][k >> 2][k & 3]));
                bad |= !__builtin_isfinite(v);
                a = fmaxf(a, v);
            }
            bmax[i] = a;
        }
        m = fmaxf(m, bmax[i]);
    }
    if (bad && nonfinite) *nonfinite = 1;
    m = wave_max_dpp(m);
    const float s = m / 2688.0f;
    const float six_s = 6.0f * s;
    if (lane == 0) tscale[r] = s;
    uint8_t *cr = codes + r * (cols / 2);
    uint8_t *sr = scales + r * (cols / 16);
    auto unpack = [&](int i, float (&v)[16]) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if constexpr (BF) {
                const uint32_t w = raw[i][k >> 2][k & 3];
                v[2 * k] = __uint_as_float(w << 16);
                v[2 * k + 1] = __uint_as_float(w & 0xFFFF0000u);
            } else {
                v[k] = __uint_as_float(raw[i][k >> 2][k & 3]);
                v[8 + k] = __uint_as_float(raw[i][2 + (k >> 2)][k & 3]);
            }
        }
    };
    // Streaming (non-temporal) stores: 8 code bytes per lane (512 contiguous bytes a
    // wave), and when a row's scale count is a multiple of 4, the scale bytes of
    // lanes 4j .. 4j + 3 gathered into one dword that lane 4j stores (every dword
    // then lies inside its row and is 4-byte aligned); byte stores otherwise.
    const bool dword_scales = (blocks & 3) == 0;
    auto store = [&](int blk, uint32_t w0, uint32_t w1, uint32_t b) {
        uint32_t sw = b;
        if (dword_scales) {
            const uint32_t b1 = __builtin_amdgcn_mov_dpp((int)b, 0x39, 0xF, 0xF, false);  // quad_perm [1,2,3,0]
            const uint32_t b2 = __builtin_amdgcn_mov_dpp((int)b, 0x4E, 0xF, 0xF, false);  // [2,3,0,1]
            const uint32_t b3 = __builtin_amdgcn_mov_dpp((int)b, 0x93, 0xF, 0xF, false);  // [3,0,1,2]
            sw = b | (b1 << 8) | (b2 << 16) | (b3 << 24);
        }
        if (blk < blocks) {
            st_nt64(w0, w1, cr + blk * 8);
            if (!dword_scales) st_nt8(b, sr + blk);
            else if ((lane & 3) == 0) st_nt32(sw, sr + blk);
        }
    };
    if (nv_fast_scale(s)) {
        const float y6 = rcp_refined(six_s);
#pragma unroll
        for (int i = 0; i < U; ++i) {
            float v[16];
            unpack(i, v);
            // E4M3 byte of the block; a byte of 0 divides by s 2^20 instead of 0, so
            // every quotient is below 2^-27 and each code is the value's sign alone
            const uint32_t b = e4m3_code_sat1(div_refined(bmax[i], six_s, y6));
            typedef float f32x2 __attribute__((ext_vector_type(2)));
            const f32x2 bv = __builtin_amdgcn_cvt_pk_f32_fp8((int)b, false);
            const float d = b ? bv[0] * s : s * 0x1p20f;
            const float y = rcp_refined(d);
            float q[2][8];
#pragma unroll
            for (int k = 0; k < 16; ++k) q[k >> 3][k & 7] = div_refined(v[k], d, y);
            store(lane + 64 * i, e2m1x8_code(q[0]), e2m1x8_code(q[1]), b);
        }
    } else {
#pragma unroll
        for (int i = 0; i < U; ++i) {
            float v[16];
            unpack(i, v);
            const uint32_t b = bmax[i] == 0.0f ? 0u : e4m3_code_sat1(bmax[i] / six_s);
            const float d = e4m3_value(b) * s;
            store(lane + 64 * i, nvfp4_codes8(v, d), nvfp4_codes8(v + 8, d), b);
        }
    }
}

// ------------------------------------------------------- NVFP4 dequantize --

// One thread per 16-block: 8 code bytes, one E4M3 byte, 16 outputs (two or four
// 16-byte stores).  E2M1 -> fp32 by the scaled FP4 conversion with scale 1
// (exact), then fl32(fl32(E2M1 * E4M3) * s), the first product exact; bf16 by
// round to nearest even.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void k_nvfp4_dequant(const uint8_t *__restrict__ codes,
                                                       const uint8_t *__restrict__ scales,
                                                       const float *__restrict__ tscale,
                                                       int per_row, uint32_t units, FastDiv cv,
                                                       int64_t cols, void *__restrict__ y,
                                                       int64_t ldy)
{
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    for (uint32_t u = blockIdx.x * 256u + threadIdx.x; u < units; u += gridDim.x * 256u) {
        const uint32_t r = fdiv(u, cv);
        const uint32_t b = u - r * cv.d;  // block within the row
        const uint2 w = *reinterpret_cast<const uint2 *>(codes + (int64_t)r * (cols / 2) + (int64_t)b * 8);
        const float bs = e4m3_value(scales[(int64_t)r * (cols / 16) + b]);
        const float s = tscale[per_row ? r : 0];
        float o[16];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const uint32_t word = q < 4 ? w.x : w.y;
            f32x2 p;
            switch (q & 3) {
            case 0: p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 0); break;
            case 1: p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 1); break;
            case 2: p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 2); break;
            default: p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 3); break;
            }
            o[2 * q] = (p[0] * bs) * s;
            o[2 * q + 1] = (p[1] * bs) * s;
        }
        const int64_t off = (int64_t)r * ldy + (int64_t)b * 16;
        if (OUT_BF16) {
            uint4 pk[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                pk[h].x = f32_to_bf16_rne(o[8 * h + 0]) | (f32_to_bf16_rne(o[8 * h + 1]) << 16);
                pk[h].y = f32_to_bf16_rne(o[8 * h + 2]) | (f32_to_bf16_rne(o[8 * h + 3]) << 16);
                pk[h].z = f32_to_bf16_rne(o[8 * h + 4]) | (f32_to_bf16_rne(o[8 * h + 5]) << 16);
                pk[h].w = f32_to_bf16_rne(o[8 * h + 6]) | (f32_to_bf16_rne(o[8 * h + 7]) << 16);
            }
            uint4 *yp = reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(y) + off);
            yp[0] = pk[0];
            yp[1] = pk[1];
        } else {
            float4 *yp = reinterpret_cast<float4 *>(reinterpret_cast<float *>(y) + off);
#pragma unroll
            for (int q = 0; q < 4; ++q) yp[q] = make_float4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
        }
    }
}

// --------------------------------------------------------- MXFP4 quantize --

// Lanes (4i .. 4i+3) hold one 32-block.  SEG writes the segment-major layout
// instead of row-major: the 64 code bytes and 4 scale bytes of row r's 128-element
// segment s at (s rows + r) * 64 and (s rows + r) * 4 (cols % 128 == 0).
template <typename T, bool SEG = false>
__global__ __launch_bounds__(256) void k_mxfp4_quant(const T *__restrict__ x, uint32_t units,
                                                     FastDiv cv, int64_t ldx, int64_t cols,
                                                     int rule, uint8_t *__restrict__ codes,
                                                     uint8_t *__restrict__ scales,
                                                     int32_t *__restrict__ nonfinite, int64_t rows = 0)
{
    int bad = 0;
    for (uint32_t u = blockIdx.x * 256u + threadIdx.x; u < units; u += gridDim.x * 256u) {
        const uint32_t r = fdiv(u, cv);
        const uint32_t c8 = u - r * cv.d;
        float v[8];
        Vec8<T>::load(x + (int64_t)r * ldx + (int64_t)c8 * 8, v);
        float bm = amax8(v, bad);
        bm = fmaxf(bm, xor1(bm));
        bm = fmaxf(bm, xor2(bm));
        uint32_t w = 0, byte = 0;
        if (bm == 0.0f) {
#pragma unroll
            for (int i = 0; i < 8; ++i) w |= ((__float_as_uint(v[i]) >> 28) & 8u) << (4 * i);
        } else {
            const int E = __builtin_amdgcn_frexp_expf(bm) - 1;        // floor(log2 bm), exact
            int k = E - 2;                                             // E2M1's top exponent is 2
            if (rule == 1 && __builtin_amdgcn_frexp_mantf(bm) > 0.75f) k = E - 1;  // 6*2^(E-2) < bm
            k = k < -127 ? -127 : (k > 127 ? 127 : k);
            byte = (uint32_t)(k + 127);
            float q[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) q[i] = __builtin_amdgcn_ldexpf(v[i], -k);  // exact
            w = e2m1x8_code(q);
        }
        if (SEG) {
            // plain stores: a lane group writes 64 bytes, half of a cache line, and as
            // streaming stores those half lines took the kernel from 28.5 to 45.5 us
            // (8192 x 5120); the row-major form writes whole lines and streams them
            const int64_t piece = (int64_t)(c8 >> 4) * rows + r;  // (segment, row)
            *reinterpret_cast<uint32_t *>(codes + piece * 64 + (c8 & 15u) * 4) = w;
            if ((c8 & 3u) == 0u) scales[piece * 4 + ((c8 >> 2) & 3u)] = (uint8_t)byte;
        } else {
            st_nt32(w, codes + (int64_t)r * (cols / 2) + (int64_t)c8 * 4);
            if ((c8 & 3u) == 0u) st_nt8(byte, scales + (int64_t)r * (cols / 32) + (c8 >> 2));
        }
    }
    if (bad && nonfinite) *nonfinite = 1;
}

// --------------------------------------------------------- MXFP8 quantize --
//
// The FP8 activations of W4A8 (edge-FP4 article, eefocus.com: an NPU with native
// W4A8, weights in FP4 and activations in FP8), read as OCP MX: 32-element blocks
// with an E8M0 scale 2^k, E4M3FN elements.  Rule 0 (OCP): k = floor(log2 amax) - 8
// (E4M3's largest exponent is 8), so the block maximum may saturate to 448;
// rule 1: the smallest k with 448 2^k >= amax.  Elements: sign | E4M3 RNE with
// saturation of |x| 2^-k (exact scaling).  Lanes (4i .. 4i+3) hold one block.
template <typename T>
__global__ __launch_bounds__(256) void k_mxfp8_quant(const T *__restrict__ x, uint32_t units,
                                                     FastDiv cv, int64_t ldx, int64_t cols,
                                                     int rule, uint8_t *__restrict__ codes,
                                                     uint8_t *__restrict__ scales,
                                                     int32_t *__restrict__ nonfinite)
{
    int bad = 0;
    for (uint32_t u = blockIdx.x * 256u + threadIdx.x; u < units; u += gridDim.x * 256u) {
        const uint32_t r = fdiv(u, cv);
        const uint32_t c8 = u - r * cv.d;
        float v[8];
        Vec8<T>::load(x + (int64_t)r * ldx + (int64_t)c8 * 8, v);
        float bm = amax8(v, bad);
        bm = fmaxf(bm, xor1(bm));
        bm = fmaxf(bm, xor2(bm));
        int k = 0;
        uint32_t byte = 0;
        if (bm != 0.0f) {
            const int E = __builtin_amdgcn_frexp_expf(bm) - 1;        // floor(log2 bm), exact
            k = E - 8;
            if (rule == 1 && __builtin_amdgcn_frexp_mantf(bm) > 0.875f) k = E - 7;  // 448*2^(E-8) < bm
            k = k < -127 ? -127 : (k > 127 ? 127 : k);
            byte = (uint32_t)(k + 127);
        }
        float a[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i] = bm == 0.0f ? 0.0f : __builtin_amdgcn_ldexpf(__builtin_fabsf(v[i]), -k);  // exact
        // the sign bits: bit 7 of each code byte (the top byte of each value)
        const uint32_t s_lo = __builtin_amdgcn_perm(__builtin_amdgcn_perm(__float_as_uint(v[3]), __float_as_uint(v[2]), 0x0c0c0703u),
                                                    __builtin_amdgcn_perm(__float_as_uint(v[1]), __float_as_uint(v[0]), 0x0c0c0703u),
                                                    0x05040100u) & 0x80808080u;
        const uint32_t s_hi = __builtin_amdgcn_perm(__builtin_amdgcn_perm(__float_as_uint(v[7]), __float_as_uint(v[6]), 0x0c0c0703u),
                                                    __builtin_amdgcn_perm(__float_as_uint(v[5]), __float_as_uint(v[4]), 0x0c0c0703u),
                                                    0x05040100u) & 0x80808080u;
        const uint32_t lo = e4m3x4_code_sat(a[0], a[1], a[2], a[3]) | s_lo;
        const uint32_t hi = e4m3x4_code_sat(a[4], a[5], a[6], a[7]) | s_hi;
        st_nt64(lo, hi, codes + (int64_t)r * cols + (int64_t)c8 * 8);
        if ((c8 & 3u) == 0u) st_nt8(byte, scales + (int64_t)r * (cols / 32) + (c8 >> 2));
    }
    if (bad && nonfinite) *nonfinite = 1;
}

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void k_mxfp4_dequant(const uint8_t *__restrict__ codes,
                                                       const uint8_t *__restrict__ scales,
                                                       uint32_t units, FastDiv cv, int64_t cols,
                                                       void *__restrict__ y, int64_t ldy)
{
    for (uint32_t u = blockIdx.x * 256u + threadIdx.x; u < units; u += gridDim.x * 256u) {
        const uint32_t r = fdiv(u, cv);
        const uint32_t c8 = u - r * cv.d;
        const uint32_t w = *reinterpret_cast<const uint32_t *>(codes + (int64_t)r * (cols / 2) + (int64_t)c8 * 4);
        const int k = (int)scales[(int64_t)r * (cols / 32) + (c8 >> 2)] - 127;
        const int64_t off = (int64_t)r * ldy + (int64_t)c8 * 8;
        if (k >= -120 && k <= 120) {
            // E2M1 times 2^k with every result normal and finite: the scaled
            // conversion applies exactly 2^k (it takes the exponent field of its
            // fp32 scale operand), 2 elements per instruction
            const float sc = __uint_as_float((uint32_t)(k + 127) << 23);
            if (OUT_BF16) {
                *reinterpret_cast<bf16x8 *>(reinterpret_cast<uint16_t *>(y) + off) = e2m1x8_bf16_pow2(w, sc);
            } else {
                typedef float f32x2 __attribute__((ext_vector_type(2)));
                const f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 0);
                const f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 1);
                const f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 2);
                const f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 3);
                float *yp = reinterpret_cast<float *>(y) + off;
                *reinterpret_cast<float4 *>(yp) = make_float4(p0[0], p0[1], p1[0], p1[1]);
                *reinterpret_cast<float4 *>(yp + 4) = make_float4(p2[0], p2[1], p3[0], p3[1]);
            }
            continue;
        }
        // the extreme scales (subnormal or overflowing results) one element at a
        // time; the E8M0 byte 0xFF encodes NaN, which every element then takes
        float o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            o[i] = k == 128 ? __uint_as_float(0x7FC00000u) : __builtin_amdgcn_ldexpf(e2m1_value(w >> (4 * i)), k);
        if (OUT_BF16) {
            uint4 p;
            p.x = f32_to_bf16_rne(o[0]) | (f32_to_bf16_rne(o[1]) << 16);
            p.y = f32_to_bf16_rne(o[2]) | (f32_to_bf16_rne(o[3]) << 16);
            p.z = f32_to_bf16_rne(o[4]) | (f32_to_bf16_rne(o[5]) << 16);
            p.w = f32_to_bf16_rne(o[6]) | (f32_to_bf16_rne(o[7]) << 16);
            *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(y) + off) = p;
        } else {
            float *yp = reinterpret_cast<float *>(y) + off;
            *reinterpret_cast<float4 *>(yp) = make_float4(o[0], o[1], o[2], o[3]);
            *reinterpret_cast<float4 *>(yp + 4) = make_float4(o[4], o[5], o[6], o[7]);
        }
    }
}

// ------------------------------------------------------------- launchers --

static unsigned grid_for(uint64_t units, unsigned cap)
{
    uint64_t g = (units + 255) / 256;
    if (g > cap) g = cap;
    return g ? (unsigned)g : 1u;
}

// The one-wave-per-row quantizer for rows of up to 8192 bf16 or 4096 fp32 values;
// false when the row is longer (the two-pass kernel takes it).
template <typename T, int U>
static void launch_rows_w(const void *x, int64_t rows, int64_t cols, int64_t ldx, uint8_t *codes, uint8_t *scales,
                          float *tscale, int32_t *nonfinite, hipStream_t st)
{
    const int64_t g = (rows + 3) / 4;
    hipLaunchKernelGGL((k_nvfp4_quant_rows_w<T, U>), dim3((unsigned)g), dim3(256), 0, st, (const T *)x, rows,
                       (int)cols, ldx, codes, scales, tscale, nonfinite);
}

static bool launch_quant_rows_w(const void *x, bool bf, int64_t rows, int64_t cols, int64_t ldx, uint8_t *codes,
                                uint8_t *scales, float *tscale, int32_t *nonfinite, hipStream_t st)
{
    const int64_t u = (cols / 16 + 63) / 64;  // 16-blocks per lane
    if ((rows + 3) / 4 > INT32_MAX || u > (bf ? 8 : 4)) return false;
#define FP4_ROWS_W(T, U) launch_rows_w<T, U>(x, rows, cols, ldx, codes, scales, tscale, nonfinite, st)
    if (bf) {
        if (u <= 1) FP4_ROWS_W(uint16_t, 1);
        else if (u <= 2) FP4_ROWS_W(uint16_t, 2);
        else if (u <= 3) FP4_ROWS_W(uint16_t, 3);
        else if (u <= 4) FP4_ROWS_W(uint16_t, 4);
        else if (u <= 5) FP4_ROWS_W(uint16_t, 5);
        else if (u <= 6) FP4_ROWS_W(uint16_t, 6);
        else FP4_ROWS_W(uint16_t, 8);
    } else {
        if (u <= 1) FP4_ROWS_W(float, 1);
        else if (u <= 2) FP4_ROWS_W(float, 2);
        else FP4_ROWS_W(float, 4);
    }
#undef FP4_ROWS_W
    return true;
}

fp4_status launch_nvfp4_quantize(const void *x, fp4_dtype xt, int64_t rows, int64_t cols,
                                 int64_t ldx, uint8_t *codes, uint8_t *scales, float *tscale,
                                 fp4_scale_mode mode, void *ws, int32_t *nonfinite,
                                 hipStream_t st)
{
    const bool bf = xt == FP4_BF16;
    if (mode == FP4_SCALE_PER_ROW && launch_quant_rows_w(x, bf, rows, cols, ldx, codes, scales, tscale, nonfinite, st))
        return hipGetLastError() == hipSuccess ? FP4_OK : FP4_ERR_HIP;
    if (mode == FP4_SCALE_PER_ROW) {
        const unsigned g = rows > 65536 ? 65536u : (unsigned)rows;
        if (bf)
            hipLaunchKernelGGL(k_nvfp4_quant_rows<uint16_t>, dim3(g), dim3(256), 0, st,
                               (const uint16_t *)x, rows, cols, ldx, codes, scales, tscale, nonfinite);
        else
            hipLaunchKernelGGL(k_nvfp4_quant_rows<float>, dim3(g), dim3(256), 0, st,
                               (const float *)x, rows, cols, ldx, codes, scales, tscale, nonfinite);
        return hipGetLastError() == hipSuccess ? FP4_OK : FP4_ERR_HIP;
    }
    const uint32_t units = (uint32_t)(rows * (cols / 8));
    const FastDiv cv = make_fastdiv((uint32_t)(cols / 8));
    const unsigned gp = grid_for(units, kAmaxPartials);
    float *partial = reinterpret_cast<float *>(ws);
    if (bf)
        hipLaunchKernelGGL(k_amax_partial<uint16_t>, dim3(gp), dim3(256), 0, st, (const uint16_t *)x,
                           units, cv, ldx, partial, nonfinite);
    else
        hipLaunchKernelGGL(k_amax_partial<float>, dim3(gp), dim3(256), 0, st, (const float *)x,
                           units, cv, ldx, partial, nonfinite);
    hipLaunchKernelGGL(k_tscale_finalize, dim3(1), dim3(256), 0, st, partial, (int)gp, tscale);
    const unsigned gq = grid_for(units, 8192);
    if (bf)
        hipLaunchKernelGGL(k_nvfp4_quant_tensor<uint16_t>, dim3(gq), dim3(256), 0, st,
                           (const uint16_t *)x, units, cv, ldx, cols, tscale, codes, scales);
    else
        hipLaunchKernelGGL(k_nvfp4_quant_tensor<float>, dim3(gq), dim3(256), 0, st,
                           (const float *)x, units, cv, ldx, cols, tscale, codes, scales);
    return hipGetLastError() == hipSuccess ? FP4_OK : FP4_ERR_HIP;
}

fp4_status launch_nvfp4_dequantize(const uint8_t *codes, const uint8_t *scales, const float *tscale,
                                   fp4_scale_mode mode, int64_t rows, int64_t cols, void *y,
                                   fp4_dtype yt, int64_t ldy, hipStream_t st)
{
    const uint32_t units = (uint32_t)(rows * (cols / 16));
    const FastDiv cv = make_fastdiv((uint32_t)(cols / 16));
    const unsigned g = grid_for(units, 16384);
    const int pr = mode == FP4_SCALE_PER_ROW;
    if (yt == FP4_BF16)
        hipLaunchKernelGGL(k_nvfp4_dequant<true>, dim3(g), dim3(256), 0, st, codes, scales, tscale,
                           pr, units, cv, cols, y, ldy);
    else
        hipLaunchKernelGGL(k_nvfp4_dequant<false>, dim3(g), dim3(256), 0, st, codes, scales, tscale,
                           pr, units, cv, cols, y, ldy);
    return hipGetLastError() == hipSuccess ? FP4_OK : FP4_ERR_HIP;
}

fp4_status launch_mxfp4_quantize(const void *x, fp4_dtype xt, int64_t rows, int64_t cols,
                                 int64_t ldx, uint8_t *codes, uint8_t *scales, fp4_mx_rule rule,
                                 int32_t *nonfinite, hipStream_t st)
{
    const uint32_t units = (uint32_t)(rows * (cols / 8));
    const FastDiv cv = make_fastdiv((uint32_t)(cols / 8));
    const unsigned g = grid_for(units, 16384);
    if (xt == FP4_BF16)
        hipLaunchKernelGGL(k_mxfp4_quant<uint16_t>, dim3(g), dim3(256), 0, st, (const uint16_t *)x,
                           units, cv, ldx, cols, (int)rule, codes, scales, nonfinite, rows);
    else
        hipLaunchKernelGGL(k_mxfp4_quant<float>, dim3(g), dim3(256), 0, st, (const float *)x,
                           units, cv, ldx, cols, (int)rule, codes, scales, nonfinite, rows);
    return hipGetLastError() == hipSuccess ? FP4_OK : FP4_ERR_HIP;
}

fp4_status launch_mxfp4_quantize_seg(const void *x, fp4_dtype xt, int64_t rows, int64_t cols,
                                     int64_t ldx, uint8_t *codes_p, uint8_t *scales_p, fp4_mx_rule rule,
                                     int32_t *nonfinite, hipStream_t st)
{
    const uint32_t units = (uint32_t)(rows * (cols / 8));
    const FastDiv cv = make_fastdiv((uint32_t)(cols / 8));
    const unsigned g = grid_for(units, 16384);
    if (xt == FP4_BF16)
        hipLaunchKernelGGL((k_mxfp4_quant<uint16_t, true>), dim3(g), dim3(256), 0, st, (const uint16_t *)x,
                           units, cv, ldx, cols, (int)rule, codes_p, scales_p, nonfinite, rows);
    else
        hipLaunchKernelGGL((k_mxfp4_quant<float, true>), dim3(g), dim3(256), 0, st, (const float *)x,
                           units, cv, ldx, cols, (int)rule, codes_p, scales_p, nonfinite, rows);
    return hipGetLastError() == hipSuccess ? FP4_OK : FP4_ERR_HIP;
}

fp4_status launch_mxfp8_quantize(const void *x, fp4_dtype xt, int64_t rows, int64_t cols,
                                 int64_t ldx, uint8_t *codes, uint8_t *scales, fp4_mx_rule rule,
                                 int32_t *nonfinite, hipStream_t st)
{
    const uint32_t units = (uint32_t)(rows * (cols / 8));
    const FastDiv cv = make_fastdiv((uint32_t)(cols / 8));
    const unsigned g = grid_for(units, 16384);
    if (xt == FP4_BF16)
        hipLaunchKernelGGL(k_mxfp8_quant<uint16_t>, dim3(g), dim3(256), 0, st, (const uint16_t *)x,
                           units, cv, ldx, cols, (int)rule, codes, scales, nonfinite);
    else
        hipLaunchKernelGGL(k_mxfp8_quant<float>, dim3(g), dim3(256), 0, st, (const float *)x,
                           units, cv, ldx, cols, (int)rule, codes, scales, nonfinite);
    return hipGetLastError() == hipSuccess ? FP4_OK : FP4_ERR_HIP;
}

fp4_status launch_mxfp4_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t rows,
                                   int64_t cols, void *y, fp4_dtype yt, int64_t ldy, hipStream_t st)
{
    const uint32_t units = (uint32_t)(rows * (cols / 8));
    const FastDiv cv = make_fastdiv((uint32_t)(cols / 8));
    const unsigned g = grid_for(units, 16384);
    if (yt == FP4_BF16)
        hipLaunchKernelGGL(k_mxfp4_dequant<true>, dim3(g), dim3(256), 0, st, codes, scales, units, cv,
                           cols, y, ldy);
    else
        hipLaunchKernelGGL(k_mxfp4_dequant<false>, dim3(g), dim3(256), 0, st, codes, scales, units,
                           cv, cols, y, ldy);
    return hipGetLastError() == hipSuccess ? FP4_OK : FP4_ERR_HIP;
}

}  // namespace fp4k
