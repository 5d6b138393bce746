// device_common.h -- gfx950 device helpers shared by the libfp4blk kernels:
// E2M1 / E4M3 / E8M0 codecs, lane reductions and small vector types.
//
// Formats: "NVFP4" (newton.com.tw wiki), section "Technical principle" (E2M1
// elements, E4M3 block scales, FP32 tensor scale); edge-FP4 article
// (eefocus.com), section "FP4 as the next core standard" (E8M0 MX scales).
// E4M3 is the OCP E4M3FN variant (bias 7, largest finite 448, no infinities).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4k {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// |q| rounded onto the E2M1 magnitudes {0,0.5,1,1.5,2,3,4,6}: each decision
// point is the midpoint of two neighbours; at a midpoint the neighbour whose
// mantissa bit is 0 (0, 1, 2, 4) wins, hence ">" at 0.25/1.25/2.5/5 and ">=" at
// 0.75/1.75/3.5.  Magnitudes above 6 saturate to index 7.  The sign bit of q
// becomes code bit 3, so a negative value rounding to 0 keeps code 0x8.
__device__ __forceinline__ uint32_t e2m1_code(float q)
{
    const float a = __builtin_fabsf(q);
    uint32_t m = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                 (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                 (uint32_t)(a > 5.0f);
    return m | ((__float_as_uint(q) >> 28) & 8u);
}

// The codes of q[0..7] (nibble i = q[i]) by gfx950's scaled FP4 conversion with
// scale 1, two values per instruction.  The conversion gives exactly e2m1_code's
// result on every non-NaN fp32 input (checked over all 2^32 bit patterns against
// e2m1_code on the device), so the quantizers use it in place of the compares.
__device__ __forceinline__ uint32_t e2m1x8_code(const float (&q)[8])
{
    uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, q[0], q[1], 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[2], q[3], 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[4], q[5], 1.0f, 2);
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[6], q[7], 1.0f, 3);
}

// Non-negative fp32 -> E4M3FN byte, round to nearest even, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_code_sat(float q)
{
    if (!(q < 448.0f)) return 0x7Eu;                            // >= 448 or +inf
    if (q < 0x1p-6f) return (uint32_t)__builtin_rintf(q * 512.0f); // subnormal: m * 2^-9, m in 0..8
    const uint32_t u = __float_as_uint(q);
    const uint32_t mant = u & 0x7FFFFFu;
    // keep 3 mantissa bits, round half to even; a carry out of the mantissa
    // lands in the exponent field by the addition below
    const uint32_t r = (mant + 0x7FFFFu + ((mant >> 20) & 1u)) >> 20;
    const uint32_t code = ((((u >> 23) & 0xFFu) - 120u) << 3) + r;  // biased exponent - 127 + 7
    return code > 0x7Eu ? 0x7Eu : code;
}

// E4M3FN bytes of four non-negative values (byte i = q_i), round to nearest even,
// saturating at 448: gfx950's scaled FP8 conversion with scale 1 on min(q, 448).
// That gives exactly e4m3_code_sat's byte for every non-negative fp32 input up to
// +inf (checked over all those bit patterns on the device; without the clamp the
// conversion returns NaN past the top of the range).
__device__ __forceinline__ uint32_t e4m3x4_code_sat(float q0, float q1, float q2, float q3)
{
    typedef short v2i16 __attribute__((ext_vector_type(2)));
    v2i16 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v2i16{0, 0}, fminf(q0, 448.0f), fminf(q1, 448.0f), 1.0f, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, fminf(q2, 448.0f), fminf(q3, 448.0f), 1.0f, true);
    return (uint32_t)(uint16_t)r[0] | ((uint32_t)(uint16_t)r[1] << 16);
}

// E4M3FN byte -> fp32 (sign honoured; 0x7F/0xFF are never produced by the quantizer).
__device__ __forceinline__ float e4m3_value(uint32_t b)
{
    const uint32_t e = (b >> 3) & 15u, m = b & 7u;
    const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
    return (b & 0x80u) ? -mag : mag;
}

// E2M1 code (4 bits) -> fp32, exact.
__device__ __forceinline__ float e2m1_value(uint32_t c)
{
    const uint32_t i = c & 7u;
    // magnitudes 0, 0.5 by index; 1..6 as 2^(e-1) * (1 + m/2) with e = i>>1, m = i&1
    const uint32_t normal_bits = (((i >> 1) + 126u) << 23) | ((i & 1u) << 22);
    const float mag = i >= 2u ? __uint_as_float(normal_bits) : (i ? 0.5f : 0.0f);
    return (c & 8u) ? -mag : mag;
}

// lane exchange with lane ^ 1 and lane ^ 2 (DPP quad permutes)
__device__ __forceinline__ float xor1(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float xor2(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
}

__device__ __forceinline__ float wave_max(float v)
{
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

// Maximum over the 64 lanes of a wave (non-negative values), returned wave-uniform:
// DPP within each row of 16 lanes, then the four row maxima read as scalars.
__device__ __forceinline__ float wave_max_dpp(float v)
{
    v = fmaxf(v, xor1(v));
    v = fmaxf(v, xor2(v));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false)));  // row_half_mirror
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false)));  // row_mirror
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// 32-bit division by a run-time constant (Granlund-Montgomery round-up method;
// exact for n, d < 2^31).
struct FastDiv {
    uint32_t d, m, s;
};

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv &f)
{
    return (__umulhi(n, f.m) + n) >> f.s;
}

// ------------------------------------------------ NVFP4 weight dequant -----

// 8 E2M1 codes (nibble i = element i) times block scale bs -> 8 bf16 (4 dwords,
// element 2i in the low half of dword i).  The hardware FP4 -> fp32 conversion
// applies only the exponent of its scale operand, so it runs with scale 1 and
// the E4M3 value is applied by an fp32 multiply.  Exact: each product has at
// most 6 significant bits, so its fp32 bits truncate to bf16 without rounding.
__device__ __forceinline__ uint4 dq8_bf16(uint32_t codes, float bs)
{
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0);
    const f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1);
    const f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2);
    const f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
    uint4 r;
    r.x = __builtin_amdgcn_perm(__float_as_uint(p0[1] * bs), __float_as_uint(p0[0] * bs), 0x07060302u);
    r.y = __builtin_amdgcn_perm(__float_as_uint(p1[1] * bs), __float_as_uint(p1[0] * bs), 0x07060302u);
    r.z = __builtin_amdgcn_perm(__float_as_uint(p2[1] * bs), __float_as_uint(p2[0] * bs), 0x07060302u);
    r.w = __builtin_amdgcn_perm(__float_as_uint(p3[1] * bs), __float_as_uint(p3[0] * bs), 0x07060302u);
    return r;
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v)
{
    bf16x8 r;
    __builtin_memcpy(&r, &v, 16);
    return r;
}

// ------------------------------------------------ MXFP4 weight dequant -----

// 8 E2M1 codes (nibble i = element i) times a power-of-two block scale -> 8 bf16.
// `scale` is the fp32 whose exponent field holds the E8M0 byte (byte << 23); the
// scaled conversion applies exactly that power of two, and E2M1 times a power of
// two is exact in bf16.
__device__ __forceinline__ bf16x8 e2m1x8_bf16_pow2(uint32_t codes, float scale)
{
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0);
    const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1);
    const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2);
    const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3);
    return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}


// E4M3FN byte (sign clear) -> fp32: the byte placed at fp32 bit 20 reads as
// 2^(e-127) (1 + m/8) (or the denormal m * 2^-129 when e == 0); times 2^120 that
// is exactly the E4M3 value (2^(e-7) (1 + m/8), or m * 2^-9).
__device__ __forceinline__ float e4m3_fast(uint32_t byte_at_bit20)
{
    return __uint_as_float(byte_at_bit20) * 0x1p120f;
}

}  // namespace fp4k
