// gemm_nv.hip -- NVFP4 GEMMs on gfx950: W4A16 decode (M <= 16), W4A16 and W4A4
// prefill (M > 16).  C = A . W^T, W [N][K] NVFP4 (codes, E4M3 block scales,
// FP32 tensor scale), blocks along K.
//
// W4A16 (Unsloth Dynamic NVFP4 article, aixq.cc, section "Core difference:
// W4A4 vs W4A16"): the 4-bit weights are widened to 16 bits and multiplied by
// 16-bit activations.  Here every weight is widened to E2M1 * E4M3 in bfloat16,
// which is exact (at most 6 significant bits, exponent range 2^-10 .. 2^11),
// so the MFMA sees the exact weight; the FP32 tensor scale is applied once in
// the fp32 epilogue.  W4A4 widens the NVFP4 activations the same way and
// multiplies by the activation row scale in the epilogue.
//
// gfx950's block-scaled FP4 matrix instruction takes a power-of-two (E8M0) scale
// per 32 K-elements; NVFP4's E4M3 scale per 16 does not fit it, so these GEMMs
// run on the bf16 MFMA (v_mfma_f32_32x32x16_bf16 / 16x16x32_bf16).
#include "device_common.h"
#include "internal.h"

namespace fp4k {

// ------------------------------------------------------------ dequant -----

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

// ------------------------------------------------------ byte-safe loads ---

template <bool ALIGNED>
__device__ __forceinline__ uint32_t ld_u32(const uint8_t *p)
{
    if (ALIGNED) return *reinterpret_cast<const uint32_t *>(p);
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}

template <bool ALIGNED>
__device__ __forceinline__ uint4 ld_u128(const uint8_t *p)
{
    if (ALIGNED) return *reinterpret_cast<const uint4 *>(p);
    uint4 r;
    r.x = ld_u32<false>(p);
    r.y = ld_u32<false>(p + 4);
    r.z = ld_u32<false>(p + 8);
    r.w = ld_u32<false>(p + 12);
    return r;
}

// ============================================================ decode =======
// M <= 16.  Workgroup = 4 waves = one 16-row N-tile (x NT); wave w owns a quarter
// of the K steps (128 K per step).  Lane l = (n = l % 16, g = l / 16) loads 32
// consecutive codes (16 bytes) of W row n at k0 + 32 g and their two scale bytes,
// and feeds them to four 16x16x32 MFMAs; MFMA j contracts the K values
// k0 + 32 g + 8 j + [0, 8) of every lane group g (a permutation of K that A and
// W share, so the sum is unchanged).  The four waves' partial tiles are added
// in LDS and the epilogue multiplies by the tensor scale.

constexpr int kDecNT = 1;  // N-tiles (16 rows) per workgroup

template <bool ALIGNED>
__global__ __launch_bounds__(256) void k_nv_decode(const uint16_t *__restrict__ a, int64_t lda,
                                                   const uint8_t *__restrict__ wc,
                                                   const uint8_t *__restrict__ wsc,
                                                   const float *__restrict__ wts, int M, int N,
                                                   int K, void *__restrict__ c, int c_bf16,
                                                   int64_t ldc)
{
    __shared__ f32x4 part[4][kDecNT][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int ln = lane & 15, g = lane >> 4;
    const int n_base = blockIdx.x * 16 * kDecNT;
    const int nsteps = (K + 127) / 128;
    const int s_begin = (nsteps * wave) / 4, s_end = (nsteps * (wave + 1)) / 4;
    const int am = ln;  // A row this lane feeds
    const bool a_ok = am < M;

    f32x4 acc[kDecNT];
#pragma unroll
    for (int t = 0; t < kDecNT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int s = s_begin; s < s_end; ++s) {
        const int kb = s * 128 + g * 32;  // first K of this lane's 32
        uint4 cw[kDecNT];
        uint32_t sw[kDecNT];
#pragma unroll
        for (int t = 0; t < kDecNT; ++t) {
            const int n = n_base + t * 16 + ln;
            cw[t] = uint4{0u, 0u, 0u, 0u};
            sw[t] = 0;
            if (n < N) {
                const uint8_t *cp = wc + (int64_t)n * (K / 2) + kb / 2;
                const uint8_t *sp = wsc + (int64_t)n * (K / 16) + kb / 16;
                if (kb + 32 <= K) {
                    cw[t] = ld_u128<ALIGNED>(cp);
                    sw[t] = ALIGNED ? (uint32_t)*reinterpret_cast<const uint16_t *>(sp)
                                    : ((uint32_t)sp[0] | ((uint32_t)sp[1] << 8));
                } else if (kb + 16 <= K) {
                    cw[t].x = ld_u32<false>(cp);
                    cw[t].y = ld_u32<false>(cp + 4);
                    sw[t] = sp[0];
                }
            }
        }
        const uint16_t *ap = a + (int64_t)am * lda + kb;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint4 av = uint4{0u, 0u, 0u, 0u};
            if (a_ok && kb + 8 * j < K) av = *reinterpret_cast<const uint4 *>(ap + 8 * j);
            const bf16x8 A = as_bf16x8(av);
#pragma unroll
            for (int t = 0; t < kDecNT; ++t) {
                const uint32_t cwj = j == 0 ? cw[t].x : j == 1 ? cw[t].y : j == 2 ? cw[t].z : cw[t].w;
                const float bs = e4m3_value((sw[t] >> (j < 2 ? 0 : 8)) & 0xFFu);
                const bf16x8 B = as_bf16x8(dq8_bf16(cwj, bs));
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc[t], 0, 0, 0);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < kDecNT; ++t) part[wave][t][lane] = acc[t];
    __syncthreads();
    const float wt = wts[0];
    // 256 threads; each (t, lane, r) output: thread -> lane = tid & 63, r = tid >> 6
    for (int idx = threadIdx.x; idx < kDecNT * 64 * 4; idx += 256) {
        const int t = idx / 256, rem = idx % 256;
        const int l = rem & 63, r = rem >> 6;
        const float v = part[0][t][l][r] + part[1][t][l][r] + part[2][t][l][r] + part[3][t][l][r];
        const int m = (l >> 4) * 4 + r;  // C row of accumulator slot r in lane l
        const int n = n_base + t * 16 + (l & 15);
        if (m < M && n < N) {
            const float o = v * wt;
            if (c_bf16)
                reinterpret_cast<uint16_t *>(c)[(int64_t)m * ldc + n] = (uint16_t)f32_to_bf16_rne(o);
            else
                reinterpret_cast<float *>(c)[(int64_t)m * ldc + n] = o;
        }
    }
}

// =========================================================== prefill =======
// 256 x 256 output tile per workgroup, 4 waves each 128 x 128 (4 x 4 tiles of
// 32 x 32), BK = 64.  Both operands are staged in LDS as bf16, row-major
// [256][64], with the 16-byte chunk c of row r stored at chunk c ^ (r & 7) so
// that MFMA fragment reads of consecutive rows hit distinct banks.  Global
// loads of step k+1 are issued before the MFMAs of step k; the widened W (and
// A for W4A4) is written to the other LDS buffer after them.

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kGroupM = 8;  // tile rows per L2 group

__device__ __forceinline__ int swz(int row, int chunk) { return row * 64 + ((chunk ^ (row & 7)) << 3); }

struct PrefetchBf16 {  // bf16 operand: 8 chunks of 16 bytes per thread
    uint4 v[8];
};
struct PrefetchFp4 {  // NVFP4 operand: one row's 64 codes + 4 scale bytes per thread
    uint4 c0, c1;
    uint32_t s;
};

template <bool ALIGNED>
__device__ __forceinline__ void load_fp4_row(PrefetchFp4 &p, const uint8_t *codes,
                                             const uint8_t *scales, int64_t row, int64_t rows,
                                             int K, int k0)
{
    p.c0 = uint4{0u, 0u, 0u, 0u};
    p.c1 = uint4{0u, 0u, 0u, 0u};
    p.s = 0;
    if (row >= rows) return;
    const uint8_t *cp = codes + row * (K / 2) + k0 / 2;
    const uint8_t *sp = scales + row * (K / 16) + k0 / 16;
    if (k0 + 64 <= K) {
        p.c0 = ld_u128<ALIGNED>(cp);
        p.c1 = ld_u128<ALIGNED>(cp + 16);
        p.s = ld_u32<ALIGNED>(sp);
    } else {
        // K tail: whole 16-blocks only (K % 16 == 0)
        uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int b = 0; b < 4; ++b) {
            if (k0 + 16 * b + 16 <= K) {
                w[2 * b] = ld_u32<false>(cp + 8 * b);
                w[2 * b + 1] = ld_u32<false>(cp + 8 * b + 4);
                p.s |= (uint32_t)sp[b] << (8 * b);
            }
        }
        p.c0 = uint4{w[0], w[1], w[2], w[3]};
        p.c1 = uint4{w[4], w[5], w[6], w[7]};
    }
}

__device__ __forceinline__ void store_fp4_row(uint16_t *lds, int row, const PrefetchFp4 &p)
{
    const uint32_t cw[8] = {p.c0.x, p.c0.y, p.c0.z, p.c0.w, p.c1.x, p.c1.y, p.c1.z, p.c1.w};
#pragma unroll
    for (int ch = 0; ch < 8; ++ch) {
        const float bs = e4m3_value((p.s >> (8 * (ch >> 1))) & 0xFFu);
        *reinterpret_cast<uint4 *>(lds + swz(row, ch)) = dq8_bf16(cw[ch], bs);
    }
}

__device__ __forceinline__ void load_bf16_tile(PrefetchBf16 &p, const uint16_t *a, int64_t lda,
                                               int64_t m0, int64_t M, int K, int k0, int tid)
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int id = i * 256 + tid;
        const int row = id >> 3, ch = id & 7;
        const int64_t m = m0 + row;
        const int k = k0 + ch * 8;
        p.v[i] = uint4{0u, 0u, 0u, 0u};
        if (m < M && k < K) p.v[i] = *reinterpret_cast<const uint4 *>(a + m * lda + k);
    }
}

__device__ __forceinline__ void store_bf16_tile(uint16_t *lds, const PrefetchBf16 &p, int tid)
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int id = i * 256 + tid;
        *reinterpret_cast<uint4 *>(lds + swz(id >> 3, id & 7)) = p.v[i];
    }
}

// Tile order: workgroups are dealt to the 8 XCDs round-robin, so workgroup b is
// renumbered to run on XCD b % 8 with consecutive logical tiles; logical tiles
// walk kGroupM tile rows before moving to the next tile column, so the
// workgroups an XCD runs together share A and W panels in its L2.
__device__ __forceinline__ void tile_of(int b, int nb, int tiles_m, int tiles_n, int &tm, int &tn)
{
    const int per = (nb + 7) / 8;
    const int xcd = b % 8, idx = b / 8;
    int logical = xcd * per + idx;
    if (nb % 8) {
        // xcd < nb % 8 own `per` slots, the rest per - 1
        const int full = nb % 8;
        logical = xcd < full ? xcd * per + idx : full * per + (xcd - full) * (per - 1) + idx;
    }
    const int group = logical / (kGroupM * tiles_n);
    const int first_m = group * kGroupM;
    const int gsz = min(kGroupM, tiles_m - first_m);
    const int in = logical % (kGroupM * tiles_n);
    tm = first_m + in % gsz;
    tn = in / gsz;
}

template <bool A_FP4, bool ALIGNED>
__global__ __launch_bounds__(256) void k_nv_gemm(NvGemmArgs g)
{
    extern __shared__ __align__(16) uint16_t smem[];
    // buffer b of A at smem + b * BM * BK, of W at smem + 2 * BM * BK + b * BN * BK
    uint16_t *const Abase = smem;
    uint16_t *const Bbase = smem + 2 * BM * BK;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int M = (int)g.M, N = (int)g.N, K = (int)g.K;
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

    PrefetchBf16 pa;
    PrefetchFp4 pa4, pw;
    const int nk = (K + BK - 1) / BK;

    // prologue
    if (A_FP4) load_fp4_row<ALIGNED>(pa4, g.a_codes, g.a_scales, m0 + tid, M, K, 0);
    else load_bf16_tile(pa, g.a, g.lda, m0, M, K, 0, tid);
    load_fp4_row<ALIGNED>(pw, g.w_codes, g.w_scales, n0 + tid, N, K, 0);
    if (A_FP4) store_fp4_row(Abase, tid, pa4);
    else store_bf16_tile(Abase, pa, tid);
    store_fp4_row(Bbase, tid, pw);
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) {
            const int k1 = (kt + 1) * BK;
            if (A_FP4) load_fp4_row<ALIGNED>(pa4, g.a_codes, g.a_scales, m0 + tid, M, K, k1);
            else load_bf16_tile(pa, g.a, g.lda, m0, M, K, k1, tid);
            load_fp4_row<ALIGNED>(pw, g.w_codes, g.w_scales, n0 + tid, N, K, k1);
        }
        const uint16_t *Ac = Abase + cur * BM * BK, *Bc = Bbase + cur * BN * BK;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int ch = ks * 2 + (lane >> 5);
            bf16x8 af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = wm * 128 + i * 32 + (lane & 31);
                af[i] = *reinterpret_cast<const bf16x8 *>(Ac + swz(row, ch));
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = wn * 128 + j * 32 + (lane & 31);
                bfr[j] = *reinterpret_cast<const bf16x8 *>(Bc + swz(row, ch));
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (more) {
            uint16_t *An = Abase + (cur ^ 1) * BM * BK, *Bn = Bbase + (cur ^ 1) * BN * BK;
            if (A_FP4) store_fp4_row(An, tid, pa4);
            else store_bf16_tile(An, pa, tid);
            store_fp4_row(Bn, tid, pw);
        }
        __syncthreads();
    }

    // epilogue: slot e of tile (i, j) is C row 32 i + 8 (e / 4) + 4 (lane / 32) + e % 4,
    // column 32 j + lane % 32 of the wave's 128 x 128 block.
    const float wt = g.w_tscale[0];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int64_t m = m0 + wm * 128 + i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
            if (m >= M) continue;
            float sc = wt;
            if (A_FP4) sc = g.a_tscale[g.a_per_row ? m : 0] * wt;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t n = n0 + wn * 128 + j * 32 + (lane & 31);
                if (n >= N) continue;
                const float o = acc[i][j][e] * sc;
                if (g.c_bf16)
                    reinterpret_cast<uint16_t *>(g.c)[m * g.ldc + n] = (uint16_t)f32_to_bf16_rne(o);
                else
                    reinterpret_cast<float *>(g.c)[m * g.ldc + n] = o;
            }
        }
    }
}

constexpr size_t kGemmLds = (size_t)2 * (BM + BN) * BK * sizeof(uint16_t);  // 128 KiB

template <bool A_FP4, bool ALIGNED>
static fp4_status launch_prefill(const NvGemmArgs &g, hipStream_t st)
{
    static bool attr_set = false;  // benign race: every setter writes the same value
    if (!attr_set) {
        if (hipFuncSetAttribute((const void *)k_nv_gemm<A_FP4, ALIGNED>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)kGemmLds) != hipSuccess)
            return FP4_ERR_HIP;
        attr_set = true;
    }
    const int tiles = (int)(((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN));
    hipLaunchKernelGGL((k_nv_gemm<A_FP4, ALIGNED>), dim3(tiles), dim3(256), kGemmLds, st, g);
    return hipGetLastError() == hipSuccess ? FP4_OK : FP4_ERR_HIP;
}

fp4_status launch_nvfp4_gemm(const NvGemmArgs &g, hipStream_t st)
{
    const bool aligned = (g.K % 64) == 0;
    if (!g.a_codes && g.M <= 16) {
        const int nwg = (int)((g.N + 16 * kDecNT - 1) / (16 * kDecNT));
        if (aligned)
            hipLaunchKernelGGL(k_nv_decode<true>, dim3(nwg), dim3(256), 0, st, g.a, g.lda, g.w_codes,
                               g.w_scales, g.w_tscale, (int)g.M, (int)g.N, (int)g.K, g.c, g.c_bf16, g.ldc);
        else
            hipLaunchKernelGGL(k_nv_decode<false>, dim3(nwg), dim3(256), 0, st, g.a, g.lda, g.w_codes,
                               g.w_scales, g.w_tscale, (int)g.M, (int)g.N, (int)g.K, g.c, g.c_bf16, g.ldc);
        return hipGetLastError() == hipSuccess ? FP4_OK : FP4_ERR_HIP;
    }
    if (g.a_codes)
        return aligned ? launch_prefill<true, true>(g, st) : launch_prefill<true, false>(g, st);
    return aligned ? launch_prefill<false, true>(g, st) : launch_prefill<false, false>(g, st);
}

}  // namespace fp4k
