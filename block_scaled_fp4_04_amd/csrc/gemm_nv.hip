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
// M <= 16, HBM-bound: the kernel's job is to keep the whole weight streaming.
// Workgroup = 4 waves over 32 W rows (two 16-row N-tiles); wave w owns a
// quarter of the K steps (128 K per step).  Lane l = (n = l % 16, g = l / 16)
// reads, for each of its steps and tiles, the 32 consecutive codes (16 bytes) of
// W row n at k0 + 32 g and their two scale bytes; all of these loads are issued
// before any arithmetic, so the full weight is in flight at once.  Each 16-byte
// run feeds four 16x16x32 MFMAs: MFMA j contracts the K values
// k0 + 32 g + 8 j + [0, 8) of every lane group g (a permutation of K that A and W
// share, so the sum is unchanged); one A fragment serves both N-tiles.  The
// four waves' partial tiles are added in LDS and the epilogue multiplies by the
// tensor scale.  At K = 5120 a wave holds its 10 steps x 2 tiles of codes in
// registers, so 544 workgroups (all resident at 3 waves per SIMD) have the whole
// weight in flight.

constexpr int kDecNT = 2;      // N-tiles (16 rows) per workgroup
constexpr int kDecWaves = 4;   // waves per workgroup, splitting K
constexpr int kDecMaxS = 10;   // K steps a wave keeps in flight

template <bool ALIGNED>
__global__ __launch_bounds__(256, 3) void k_nv_decode_generic(const uint16_t *__restrict__ a, int64_t lda,
                                                   const uint8_t *__restrict__ wc,
                                                   const uint8_t *__restrict__ wsc,
                                                   const float *__restrict__ wts, int M, int N,
                                                   int K, void *__restrict__ c, int c_bf16,
                                                   int64_t ldc)
{
    __shared__ f32x4 part[kDecWaves][kDecNT][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int ln = lane & 15, g = lane >> 4;
    const int n_base = blockIdx.x * 16 * kDecNT;
    const int nsteps = (K + 127) / 128;
    const int s_begin = (nsteps * wave) / kDecWaves, s_end = (nsteps * (wave + 1)) / kDecWaves;
    const bool a_ok = ln < M;
    const uint16_t *arow = a + (int64_t)(a_ok ? ln : 0) * lda;

    f32x4 acc[kDecNT];
#pragma unroll
    for (int t = 0; t < kDecNT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int s0 = s_begin; s0 < s_end; s0 += kDecMaxS) {
        const int ns = min(kDecMaxS, s_end - s0);
        uint4 cw[kDecMaxS][kDecNT];
        uint32_t sw[kDecMaxS][kDecNT];
        // issue every weight load of this chunk first
#pragma unroll
        for (int i = 0; i < kDecMaxS; ++i) {
#pragma unroll
            for (int t = 0; t < kDecNT; ++t) {
                cw[i][t] = uint4{0u, 0u, 0u, 0u};
                sw[i][t] = 0;
                const int n = n_base + t * 16 + ln;
                const int kb = (s0 + i) * 128 + g * 32;
                if (i < ns && n < N) {
                    const uint8_t *cp = wc + (int64_t)n * (K / 2) + kb / 2;
                    const uint8_t *sp = wsc + (int64_t)n * (K / 16) + kb / 16;
                    if (kb + 32 <= K) {
                        cw[i][t] = ld_u128<ALIGNED>(cp);
                        sw[i][t] = ALIGNED ? (uint32_t)*reinterpret_cast<const uint16_t *>(sp)
                                           : ((uint32_t)sp[0] | ((uint32_t)sp[1] << 8));
                    } else if (kb + 16 <= K) {
                        cw[i][t].x = ld_u32<false>(cp);
                        cw[i][t].y = ld_u32<false>(cp + 4);
                        sw[i][t] = sp[0];
                    }
                }
            }
        }
#pragma unroll
        for (int i = 0; i < kDecMaxS; ++i) {
            if (i < ns) {
                const int kb = (s0 + i) * 128 + g * 32;
                float bs[kDecNT][2];
#pragma unroll
                for (int t = 0; t < kDecNT; ++t) {
                    bs[t][0] = e4m3_value(sw[i][t] & 0xFFu);
                    bs[t][1] = e4m3_value((sw[i][t] >> 8) & 0xFFu);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    uint4 av = uint4{0u, 0u, 0u, 0u};
                    if (a_ok && kb + 8 * j < K) av = *reinterpret_cast<const uint4 *>(arow + kb + 8 * j);
                    const bf16x8 A = as_bf16x8(av);
#pragma unroll
                    for (int t = 0; t < kDecNT; ++t) {
                        const uint32_t cwj = j == 0 ? cw[i][t].x : j == 1 ? cw[i][t].y : j == 2 ? cw[i][t].z : cw[i][t].w;
                        const bf16x8 B = as_bf16x8(dq8_bf16(cwj, bs[t][j >> 1]));
                        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc[t], 0, 0, 0);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < kDecNT; ++t) part[wave][t][lane] = acc[t];
    __syncthreads();
    const float wt = wts[0];
    // kDecNT * 64 lanes * 4 slots outputs; slot r of lane l is C row 4 (l / 16) + r,
    // column l % 16 of the tile
    for (int idx = threadIdx.x; idx < kDecNT * 256; idx += 64 * kDecWaves) {
        const int t = idx >> 8, rem = idx & 255;
        const int l = rem & 63, r = rem >> 6;
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < kDecWaves; ++w) v += part[w][t][l][r];
        const int m = (l >> 4) * 4 + r;
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

// Decode kernel for K % 128 == 0 (the common case).  Workgroup = 4 waves on 16
// W rows; wave w owns a quarter of the K steps and walks it in passes of up to
// 5 steps (640 K).  A pass's codes are read with coalesced 16-byte loads -- the
// 64 lanes cover consecutive 16-byte chunks of the 16 rows' pass segments -- and
// its scale bytes with coalesced 32-bit loads; the wave then writes them to its
// own LDS region in the order the MFMA wants and reads them back (no other wave
// touches that region, so a wave-scope fence is the only synchronization).  The
// chunk of row r holding K values [32 c, 32 c + 32) of the pass feeds MFMA
// lane r + 16 (c % 4) in step c / 4: a permutation of K shared with A.  Loads of
// pass p + 1 are issued before pass p is computed.

constexpr int kDecP = 5;                      // steps (128 K) per pass
constexpr int kDecChunks = kDecP * 4 * 16 / 64;   // 16-byte code chunks per lane per pass = 5
constexpr int kDecSDw = (kDecP * 8 * 16 + 255) / 256;  // scale dwords per lane per pass = 3

struct DecPass {
    u32x4 c[kDecChunks];
    uint32_t s[kDecSDw];
};

__device__ __forceinline__ void dec_load(DecPass &p, const uint8_t *__restrict__ wc,
                                         const uint8_t *__restrict__ wsc, int n0, int N, int K,
                                         int kpass, int steps, int lane)
{
    const int seg = steps * 4;  // 16-byte chunks per row in this pass
#pragma unroll
    for (int i = 0; i < kDecChunks; ++i) {
        const int q = i * 64 + lane;
        const int row = q / (kDecP * 4), c = q % (kDecP * 4);
        p.c[i] = u32x4{0u, 0u, 0u, 0u};
        if (c < seg && n0 + row < N)
            p.c[i] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4 *>(wc + (int64_t)(n0 + row) * (K / 2) + kpass / 2) + c);
    }
    // scale bytes of the pass: 16 rows x (steps * 8) bytes, as dwords
    const int sdw = steps * 2;  // dwords per row
#pragma unroll
    for (int i = 0; i < kDecSDw; ++i) {
        const int q = i * 64 + lane;
        const int row = q / (kDecP * 2), d = q % (kDecP * 2);
        p.s[i] = 0;
        if (row < 16 && d < sdw && n0 + row < N)
            p.s[i] = reinterpret_cast<const uint32_t *>(wsc + (int64_t)(n0 + row) * (K / 16) + kpass / 16)[d];
    }
}

__device__ __forceinline__ void dec_stage(uint8_t *lds, const DecPass &p, int lane)
{
    // codes: chunk (row, c) -> slot (c / 4) * 64 + row + 16 (c % 4); scales: [row][kDecP * 8]
#pragma unroll
    for (int i = 0; i < kDecChunks; ++i) {
        const int q = i * 64 + lane;
        const int row = q / (kDecP * 4), c = q % (kDecP * 4);
        reinterpret_cast<u32x4 *>(lds)[(c >> 2) * 64 + row + 16 * (c & 3)] = p.c[i];
    }
#pragma unroll
    for (int i = 0; i < kDecSDw; ++i) {
        const int q = i * 64 + lane;
        if (q < 16 * kDecP * 2) reinterpret_cast<uint32_t *>(lds + kDecP * 64 * 16)[q] = p.s[i];
    }
}


// One pass of the decode kernel over `steps` (compile-time) steps.
template <int STEPS>
__device__ __forceinline__ void dec_compute(f32x4 &acc, const uint8_t *lds, const uint16_t *arow,
                                            int kpass, int lane, int i0)
{
    const int ln = lane & 15, g = lane >> 4;
    const uint32_t *sp = reinterpret_cast<const uint32_t *>(lds + kDecP * 64 * 16);
#pragma unroll
    for (int ii = 0; ii < STEPS; ++ii) {
        const int i = i0 + ii;
        const u32x4 cw = reinterpret_cast<const u32x4 *>(lds)[i * 64 + lane];
        // scale bytes of this lane's two 16-blocks: row ln, bytes 8 i + 2 g, 8 i + 2 g + 1
        const uint32_t sw = sp[ln * (kDecP * 2) + 2 * i + (g >> 1)] >> (16 * (g & 1));
        const float bs0 = e4m3_fast((sw << 20) & 0x0FF00000u);
        const float bs1 = e4m3_fast((sw << 12) & 0x0FF00000u);
        const uint16_t *ap = arow + kpass + i * 128 + g * 32;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bf16x8 A = *reinterpret_cast<const bf16x8 *>(ap + 8 * j);
            const bf16x8 B = as_bf16x8(dq8_bf16(cw[j], j < 2 ? bs0 : bs1));
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc, 0, 0, 0);
        }
    }
}

__device__ __forceinline__ void dec_pass(f32x4 &acc, uint8_t *lds, const DecPass &p,
                                         const uint16_t *arow, int kpass, int steps, int lane)
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    dec_stage(lds, p, lane);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (steps == kDecP) {
        dec_compute<kDecP>(acc, lds, arow, kpass, lane, 0);
    } else {
        for (int i = 0; i < steps; ++i) dec_compute<1>(acc, lds, arow, kpass, lane, i);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
}

__global__ __launch_bounds__(256) void k_nv_decode(const uint16_t *__restrict__ a, int64_t lda,
                                                   const uint8_t *__restrict__ wc,
                                                   const uint8_t *__restrict__ wsc,
                                                   const float *__restrict__ wts, int M, int N,
                                                   int K, void *__restrict__ c, int c_bf16,
                                                   int64_t ldc)
{
    constexpr int kRegion = kDecP * 64 * 16 + 16 * kDecP * 8;  // codes + scale bytes per wave
    __shared__ __align__(16) uint8_t stage[4][kRegion];
    __shared__ f32x4 part[4][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int ln = lane & 15;
    const int n0 = blockIdx.x * 16;
    const int nsteps = K / 128;
    const int s_begin = (nsteps * wave) / 4, s_end = (nsteps * (wave + 1)) / 4;
    // lanes feeding A rows >= M read row M - 1 instead: those MFMA output rows are
    // never stored, and no other output row depends on them
    const uint16_t *arow = a + (int64_t)min(ln, M - 1) * lda;
    uint8_t *lds = stage[wave];

    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    DecPass p0, p1;
    int s0 = s_begin;
    if (s0 < s_end) dec_load(p0, wc, wsc, n0, N, K, s0 * 128, min(kDecP, s_end - s0), lane);
    while (s0 < s_end) {
        const int st0 = min(kDecP, s_end - s0);
        const int s1 = s0 + st0;
        if (s1 < s_end) dec_load(p1, wc, wsc, n0, N, K, s1 * 128, min(kDecP, s_end - s1), lane);
        dec_pass(acc, lds, p0, arow, s0 * 128, st0, lane);
        if (s1 >= s_end) break;
        const int st1 = min(kDecP, s_end - s1);
        const int s2 = s1 + st1;
        if (s2 < s_end) dec_load(p0, wc, wsc, n0, N, K, s2 * 128, min(kDecP, s_end - s2), lane);
        dec_pass(acc, lds, p1, arow, s1 * 128, st1, lane);
        s0 = s2;
    }
    part[wave][lane] = acc;
    __syncthreads();
    const float wt = wts[0];
    {
        const int l = threadIdx.x & 63, r = threadIdx.x >> 6;
        const float v = part[0][l][r] + part[1][l][r] + part[2][l][r] + part[3][l][r];
        const int m = (l >> 4) * 4 + r;
        const int n = n0 + (l & 15);
        if (m < M && n < N) {
            const float o = v * wt;
            if (c_bf16)
                reinterpret_cast<uint16_t *>(c)[(int64_t)m * ldc + n] = (uint16_t)f32_to_bf16_rne(o);
            else
                reinterpret_cast<float *>(c)[(int64_t)m * ldc + n] = o;
        }
    }
}

// Persistent decode kernel for K = 1024 S (S = 1..8 steps of 128 K per wave).
// One workgroup per CU, 8 waves; workgroup b owns W rows [N b / G, N (b+1) / G),
// so every CU streams the same number of weight bytes.  Wave w owns K slice
// [128 S w, 128 S (w+1)): it loads its A fragments once (S x 4 16-byte loads per
// lane, kept in registers for the whole kernel) and then walks the workgroup's
// 16-row tiles.  A tile's codes and scale bytes for the slice are copied into a
// per-wave LDS ring (depth D) by global->LDS DMA loads that read whole 128-byte
// lines: instruction t, lane i fetches row-major chunk 64 t + (i ^ ((i >> 4) & 3))
// of the tile (16 rows x 4 S chunks of 16 bytes) and lands in LDS slot 64 t + i.
// The MFMA lane (n, g) then reads chunk (n, 4 s + g) at slot 64 t + (o ^ ((o >> 4)
// & 3)) (o = q % 64, t = q / 64, q = 4 S n + 4 s + g), which for odd S puts the 16
// lanes of a group on 16 different bank groups.  The ring keeps D - 1 tiles in
// flight; waits are exact vmcnt counts of the DMA loads issued after the tile
// being consumed.  The eight K-slice partial tiles are summed in LDS at the end.

constexpr int kPersistWaves = 8;
constexpr int kPersistMaxT = 5;   // 16-row tiles per workgroup

__device__ __forceinline__ void waitcnt_vm(int n)
{
    // s_waitcnt with vmcnt = n (n < 64), expcnt and lgkmcnt left at their maxima
    switch (n) {
#define FP4K_WC(N) case N: __builtin_amdgcn_s_waitcnt(((N) & 0xF) | (((N) >> 4) << 14) | (0x7 << 4) | (0xF << 8)); break;
        FP4K_WC(0) FP4K_WC(1) FP4K_WC(2) FP4K_WC(3) FP4K_WC(4) FP4K_WC(5) FP4K_WC(6) FP4K_WC(7)
        FP4K_WC(8) FP4K_WC(9) FP4K_WC(10) FP4K_WC(11) FP4K_WC(12) FP4K_WC(13) FP4K_WC(14) FP4K_WC(15)
        FP4K_WC(16) FP4K_WC(17) FP4K_WC(18) FP4K_WC(19) FP4K_WC(20) FP4K_WC(21) FP4K_WC(22) FP4K_WC(23)
        FP4K_WC(24) FP4K_WC(25) FP4K_WC(26) FP4K_WC(27) FP4K_WC(28) FP4K_WC(29) FP4K_WC(30) FP4K_WC(31)
#undef FP4K_WC
    default: __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8)); break;  // vmcnt(0)
    }
}

template <int S>
struct PersistCfg {
    static constexpr int kCodeBytes = 16 * S * 64;               // 16 rows x S steps x 64 bytes
    static constexpr int kCodeInstr = kCodeBytes / 1024;         // 16-byte DMA instructions = S
    static constexpr int kScaleDw = 16 * S * 2;                  // scale dwords of a tile slice
    static constexpr int kScaleInstr = (kScaleDw + 63) / 64;     // 4-byte DMA instructions
    static constexpr int kUnitBytes = kCodeBytes + kScaleInstr * 256;
    static constexpr int D = S <= 5 ? 3 : 2;                     // ring depth (tiles)
    static constexpr int kLoads = kCodeInstr + kScaleInstr;      // vmem instructions per tile
    static constexpr size_t kRing = (size_t)kPersistWaves * D * kUnitBytes;
    static constexpr size_t kReduce = (size_t)kPersistWaves * kPersistMaxT * 64 * 16;  // partial tiles
    static constexpr size_t kLds = kRing > kReduce ? kRing : kReduce;
};

typedef __attribute__((address_space(3))) void lds_void;

// Per-lane byte offsets of a tile's DMA sources, relative to the tile's first row
// (computed once; a tile adds a wave-uniform base).
template <int S>
struct PersistLane {
    uint32_t code_off[PersistCfg<S>::kCodeInstr];
    uint32_t scale_off[PersistCfg<S>::kScaleInstr];
    uint8_t code_row[PersistCfg<S>::kCodeInstr];
    uint8_t scale_row[PersistCfg<S>::kScaleInstr];
};

template <int S>
__device__ __forceinline__ void persist_lane_init(PersistLane<S> &pl, int K, int kslice, int lane)
{
    using C = PersistCfg<S>;
    const int o = lane ^ ((lane >> 4) & 3);
#pragma unroll
    for (int t = 0; t < C::kCodeInstr; ++t) {
        const int q = 64 * t + o;
        const int row = q / (4 * S), cc = q % (4 * S);
        pl.code_row[t] = (uint8_t)row;
        pl.code_off[t] = (uint32_t)(row * (K / 2) + kslice / 2 + cc * 16);
    }
#pragma unroll
    for (int t = 0; t < C::kScaleInstr; ++t) {
        const int q = min(64 * t + lane, C::kScaleDw - 1);
        const int row = q / (2 * S), d = q % (2 * S);
        pl.scale_row[t] = (uint8_t)row;
        pl.scale_off[t] = (uint32_t)(row * (K / 16) + kslice / 16 + 4 * d);
    }
}

// DMA one tile (rows t0 .. t0 + 15, clamped to n_hi - 1) of the wave's K slice into buf.
// The weight copies carry the non-temporal hint (cache policy 2): each weight byte
// is read once per call.
template <int S>
__device__ __forceinline__ void persist_issue(uint8_t *buf, const uint8_t *__restrict__ wc,
                                              const uint8_t *__restrict__ wsc, int t0, int n_hi,
                                              int K, const PersistLane<S> &pl)
{
    using C = PersistCfg<S>;
    const uint8_t *cbase = wc + (int64_t)t0 * (K / 2);
    const uint8_t *sbase = wsc + (int64_t)t0 * (K / 16);
    if (t0 + 16 <= n_hi) {
#pragma unroll
        for (int t = 0; t < C::kCodeInstr; ++t)
            __builtin_amdgcn_global_load_lds(cbase + pl.code_off[t], (lds_void *)(buf + t * 1024), 16, 0, 2);
#pragma unroll
        for (int t = 0; t < C::kScaleInstr; ++t)
            __builtin_amdgcn_global_load_lds(sbase + pl.scale_off[t],
                                             (lds_void *)(buf + C::kCodeBytes + t * 256), 4, 0, 2);
    } else {
        // partial last tile: rows past n_hi re-read row n_hi - 1 (never stored)
        const int last = n_hi - 1 - t0;
#pragma unroll
        for (int t = 0; t < C::kCodeInstr; ++t) {
            const int back = max((int)pl.code_row[t] - last, 0);
            __builtin_amdgcn_global_load_lds(cbase + pl.code_off[t] - (int64_t)back * (K / 2),
                                             (lds_void *)(buf + t * 1024), 16, 0, 2);
        }
#pragma unroll
        for (int t = 0; t < C::kScaleInstr; ++t) {
            const int back = max((int)pl.scale_row[t] - last, 0);
            __builtin_amdgcn_global_load_lds(sbase + pl.scale_off[t] - (int64_t)back * (K / 16),
                                             (lds_void *)(buf + C::kCodeBytes + t * 256), 4, 0, 2);
        }
    }
}

template <int S>
__global__ __launch_bounds__(512, 1) void k_nv_decode_persist(const uint16_t *__restrict__ a,
                                                              int64_t lda,
                                                              const uint8_t *__restrict__ wc,
                                                              const uint8_t *__restrict__ wsc,
                                                              const float *__restrict__ wts, int M,
                                                              int N, int K, void *__restrict__ c,
                                                              int c_bf16, int64_t ldc)
{
    using C = PersistCfg<S>;
    extern __shared__ __align__(16) uint8_t psmem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ln = lane & 15, g = lane >> 4;
    const int n_lo = (int)((int64_t)N * blockIdx.x / gridDim.x);
    const int n_hi = (int)((int64_t)N * (blockIdx.x + 1) / gridDim.x);
    const int ntiles = (n_hi - n_lo + 15) / 16;
    const int kslice = wave * S * 128;
    uint8_t *ring = psmem + (size_t)wave * C::D * C::kUnitBytes;

    // A fragments of this wave's K slice (rows >= M read row M - 1: their MFMA
    // output rows are never stored and no stored row depends on them)
    bf16x8 af[S][4];
    {
        const uint16_t *ap = a + (int64_t)min(ln, M - 1) * lda + kslice + g * 32;
#pragma unroll
        for (int s = 0; s < S; ++s)
#pragma unroll
            for (int j = 0; j < 4; ++j) af[s][j] = *reinterpret_cast<const bf16x8 *>(ap + s * 128 + j * 8);
    }
    PersistLane<S> pl;
    persist_lane_init<S>(pl, K, kslice, lane);
    if (ntiles > 0) persist_issue<S>(ring, wc, wsc, n_lo, n_hi, K, pl);
    if (C::D > 2 && ntiles > 1) persist_issue<S>(ring + C::kUnitBytes, wc, wsc, n_lo + 16, n_hi, K, pl);

    // LDS offsets this lane reads: code slot of step s, scale dword and shift
    uint32_t code_slot[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int q = 4 * S * ln + 4 * s + g;
        code_slot[s] = (uint32_t)(((q & ~63) | ((q & 63) ^ (((q & 63) >> 4) & 3))) * 16);
    }
    const uint32_t scale_base = (uint32_t)(C::kCodeBytes + (ln * 2 * S + (g >> 1)) * 4);
    const uint32_t scale_shift = 16u * (g & 1);

    f32x4 acc[kPersistMaxT];
#pragma unroll
    for (int u = 0; u < kPersistMaxT; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int u = 0; u < kPersistMaxT; ++u) {
        if (u < ntiles) {
            const int ahead = u + C::D - 1;  // tile issued now, into the slot tile u - 1 used
            __builtin_amdgcn_s_waitcnt((0x3F & 0xF) | (0x3 << 14) | (0x7 << 4));  // lgkmcnt(0)
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            if (ahead < ntiles)
                persist_issue<S>(ring + (ahead % C::D) * C::kUnitBytes, wc, wsc, n_lo + 16 * ahead, n_hi,
                                 K, pl);
            // tiles issued after tile u: min(D - 1, ntiles - 1 - u)
            waitcnt_vm(min(C::D - 1, ntiles - 1 - u) * C::kLoads);
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const uint8_t *buf = ring + (u % C::D) * C::kUnitBytes;
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const u32x4 cw = *reinterpret_cast<const u32x4 *>(buf + code_slot[s]);
                const uint32_t sw = *reinterpret_cast<const uint32_t *>(buf + scale_base + 8 * s) >> scale_shift;
                const float bs0 = e4m3_fast((sw << 20) & 0x0FF00000u);
                const float bs1 = e4m3_fast((sw << 12) & 0x0FF00000u);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bf16x8 B = as_bf16x8(dq8_bf16(cw[j], j < 2 ? bs0 : bs1));
                    acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s][j], B, acc[u], 0, 0, 0);
                }
            }
        }
    }

    // sum the eight K-slice partials (the rings are free now)
    __syncthreads();
    f32x4 *part = reinterpret_cast<f32x4 *>(psmem);  // [wave][tile][lane]
#pragma unroll
    for (int u = 0; u < kPersistMaxT; ++u)
        if (u < ntiles) part[(wave * kPersistMaxT + u) * 64 + lane] = acc[u];
    __syncthreads();
    const float wt = wts[0];
    for (int idx = threadIdx.x; idx < ntiles * 256; idx += 64 * kPersistWaves) {
        const int u = idx >> 8, l = idx & 63, r = (idx >> 6) & 3;
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < kPersistWaves; ++w) v += part[(w * kPersistMaxT + u) * 64 + l][r];
        const int m = (l >> 4) * 4 + r;
        const int n = n_lo + 16 * u + (l & 15);
        if (m < M && n < n_hi) {
            const float o = v * wt;
            if (c_bf16)
                reinterpret_cast<uint16_t *>(c)[(int64_t)m * ldc + n] = (uint16_t)f32_to_bf16_rne(o);
            else
                reinterpret_cast<float *>(c)[(int64_t)m * ldc + n] = o;
        }
    }
}

template <int S>
static fp4_status launch_decode_persist(const NvGemmArgs &g, hipStream_t st)
{
    using C = PersistCfg<S>;
    static std::atomic<uint64_t> lds_set{0};  // per device
    if (!set_max_lds_once((const void *)k_nv_decode_persist<S>, (int)C::kLds, lds_set)) return FP4_ERR_HIP;
    // enough workgroups that none owns more than kPersistMaxT tiles, at least one per CU
    int64_t grid = (g.N + 16 * kPersistMaxT - 1) / (16 * kPersistMaxT);
    if (grid < 256) grid = 256;
    if (grid > (g.N + 15) / 16) grid = (g.N + 15) / 16;
    hipLaunchKernelGGL(k_nv_decode_persist<S>, dim3((unsigned)grid), dim3(64 * kPersistWaves), C::kLds,
                       st, g.a, g.lda, g.w_codes, g.w_scales, g.w_tscale, (int)g.M, (int)g.N, (int)g.K,
                       g.c, g.c_bf16, g.ldc);
    return hipGetLastError() == hipSuccess ? FP4_OK : FP4_ERR_HIP;
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

// ---------------------------------------------- prefill, DMA ring (K % 64) --
//
// TM x TN output tile (256 x 256, or 128 x 128 for a last partial round), four
// waves, built around what moves:
//  - Operands travel HBM -> LDS by buffer-to-LDS DMA, in their stored form: bf16
//    A tiles (W4A16) or packed codes + E4M3 bytes (W4A4 A, and W always).  LDS
//    holds W at 4.5 bits a value, not widened, so a 256 x 256 stage is 41 KiB
//    (W4A16) or 18 KiB (W4A4) and three stages are in flight.
//  - W may also come in the decode layout (segment-major, see nvfp4_pack_decode):
//    a stage's W panel is then one half of each row's 64-byte segment piece, 256
//    rows 64 bytes apart, instead of 32-byte pieces of 256 separate rows.
//  - Each wave widens the W (and W4A4 A) fragments it multiplies straight from
//    LDS into registers (exact E2M1 x E4M3 in bf16), between MFMAs.
//  - The K order inside a 64-element stage is permuted the same way for both
//    operands: MFMA step ks, lane half h contracts K = 32 h + 8 ks + [0, 8), so a
//    lane's 16 code bytes of a row feed its four steps.
//  - MFMA computes W_j A_i^T, so each lane ends with 4 consecutive output columns
//    of one row, which the epilogue stages through LDS into whole-row stores.
// Stages are three separate LDS objects (the compiler then never waits for a DMA
// into one before reading another), rotated by unrolling the K loop 3 times, with
// the last K % 3 stages peeled; copies of stages past K go through size-0
// descriptors (zeros, nothing read).
constexpr int kRK = 64;  // K elements per stage
// 8 E2M1 codes times one E4M3 block scale -> 8 fp16, exact.  An E2M1 magnitude
// has at most 2 significant bits and an E4M3 value at most 4, so their product
// has at most 6 (fp16 keeps 11), and it lies in [2^-10, 2688], inside fp16's
// normal range: the packed fp16 multiply never rounds.  (bf16 would hold the
// product too, but gfx950 has no packed bf16 multiply: the bf16 form above
// multiplies in fp32 and packs, 16 VALU per 8 elements against 8 here.)
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ uint4 dq8_f16(uint32_t codes, _Float16 bs)
{
    const f16x2 s = {bs, bs};
    const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * s;
    const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * s;
    const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * s;
    const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * s;
    uint4 r;
    __builtin_memcpy(&r.x, &p0, 4);
    __builtin_memcpy(&r.y, &p1, 4);
    __builtin_memcpy(&r.z, &p2, 4);
    __builtin_memcpy(&r.w, &p3, 4);
    return r;
}

// Operand formats of the ring kernel (template parameter F): W4A16 with NVFP4
// weights, W4A4 with NVFP4 on both sides, W4A16 with MXFP4 weights.
constexpr int kFmtNv16 = 0, kFmtNv44 = 1, kFmtMx16 = 2;
constexpr int kNvL16 = 1;  // wave layout of the W4A16 256 x 256 tile (see NvTile)

// Tile geometry.  Wave layout L = 0 splits the tile 2 x 2; L = 1 splits N four
// ways (each wave all TM rows), so no two waves widen the same W rows.
template <bool A_FP4, int L, int TM, int TN>
struct NvTile {
    static_assert((TM == 128 || TM == 256) && (TN == 128 || TN == 256), "tile");
    static constexpr int WM = L ? TM : TM / 2;      // rows per wave
    static constexpr int WN = L ? TN / 4 : TN / 2;  // columns per wave
    static constexpr int NI = WM / 32, NJ = WN / 32;
    static_assert(NI * 32 == WM && NJ * 32 == WN && NJ >= 1, "wave tile");
    __device__ static int row0(int wave) { return L ? 0 : (wave >> 1) * WM; }
    __device__ static int col0(int wave) { return L ? WN * wave : (wave & 1) * WN; }
    // byte offsets inside a stage
    static constexpr int kA = 0;                             // bf16 [TM][64] or codes [TM][32]
    static constexpr int kAS = A_FP4 ? TM * 32 : 0;          // A scales [TM][4] (W4A4)
    static constexpr int kW = A_FP4 ? kAS + TM * 4 : TM * 128;  // W codes [TN][32]
    static constexpr int kWS = kW + TN * 32;                 // W scales [TN][4]
    static constexpr int kUsed = kWS + TN * 4;
    // copies per wave per stage: 16-byte chunks (8 per bf16 row, 2 per packed
    // row) and one 4-byte scale word per row
    static constexpr int nA = A_FP4 ? TM * 2 / 256 : TM * 8 / 256;
    static constexpr int nW = TN * 2 / 256;
    static constexpr int kDma = nA + nW + 1 + (A_FP4 ? 1 : 0);
    // epilogue: the two row halves of the tile are staged through two stage
    // buffers, R rows at a time (rows padded by 16 bytes).  128 x 256 tiles stage
    // 32 rows a round, so that their stage stays at the size the K loop needs and
    // two workgroups fit in a CU's LDS (bf16 output)
    static constexpr int H = TM / 2;
    static constexpr bool kTwoPerCu = TM == 128 && TN == 256;
    static constexpr int epi_rows(int es) { return kTwoPerCu ? 32 : (es == 2 ? 64 : 32) < H ? (es == 2 ? 64 : 32) : H; }
    static constexpr int epi_pitch(int es) { return TN * es + 16; }
    static constexpr int stage_bytes(int es)
    {
        return kUsed > epi_rows(es) * epi_pitch(es) ? kUsed : epi_rows(es) * epi_pitch(es);
    }
};

struct NvRingDma {
    __amdgpu_buffer_rsrc_t ra, ras, rw, rws;
    uint32_t a[8], as, w[2], ws;
    // W in the decode layout: a 128-element segment's codes and scale bytes of all
    // weight rows are seg_w and seg_s bytes; stage k0 is half (k0 / 64) % 2 of
    // segment k0 / 128
    int seg;
    uint32_t seg_w, seg_s;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t nv_rsrc(const void *base, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)(uint32_t)bytes, 0x00020000);
}

typedef __attribute__((address_space(3))) void nv_lds_void;
constexpr uint32_t kNvOut = 0x80000000u;  // an offset past every descriptor's size

// Copy-lane assignment.  16-byte chunk q of a wave's share: codes chunk h of row
// r lands at 32 r + 16 (h ^ ((r >> 3) & 1)); bf16 chunk c of A row r at
// 128 r + 16 (c ^ ((r >> 1) & 7)): conflict-free 16-lane fragment reads.  Scale
// word of row r at 4 r; with fewer than 256 rows the upper waves repeat the lower
// waves' rows (same bytes to the same place).
template <int F, int L, int TM, int TN>
__device__ __forceinline__ void nv_ring_dma(uint8_t *st, const NvRingDma &d, int k0, int wave)
{
    using S = NvTile<F == 1, L, TM, TN>;
    constexpr bool A_FP4 = F == kFmtNv44;
    if constexpr (A_FP4) {
#pragma unroll
        for (int i = 0; i < S::nA; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                d.ra, (nv_lds_void *)(st + S::kA + 16 * (64 * S::nA * wave + 64 * i)), 16, (int)d.a[i], k0 / 2, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(d.ras, (nv_lds_void *)(st + S::kAS + 256 * (wave % (TM / 64))), 4,
                                                 (int)d.as, k0 / 16, 0, 0);
    } else {
#pragma unroll
        for (int i = 0; i < S::nA; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                d.ra, (nv_lds_void *)(st + S::kA + 16 * (64 * S::nA * wave + 64 * i)), 16, (int)d.a[i], 2 * k0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < S::nW; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            d.rw, (nv_lds_void *)(st + S::kW + 16 * (64 * S::nW * wave + 64 * i)), 16, (int)d.w[i],
            d.seg ? (int)((k0 >> 7) * d.seg_w + ((k0 >> 6) & 1) * 32) : k0 / 2, 0, 0);
    // NVFP4: the row's 4 E4M3 bytes of the stage.  MXFP4: the aligned dword holding
    // the row's 2 E8M0 bytes of the stage (the two bytes of stage pair t / 2;
    // K % 128 == 0 keeps it inside the row).
    const int ks_off = d.seg ? (int)((k0 >> 7) * d.seg_s + (F == kFmtMx16 ? 0 : ((k0 >> 6) & 1) * 4))
                             : F == kFmtMx16 ? ((k0 / kRK) & ~1) * 2 : k0 / 16;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rws, (nv_lds_void *)(st + S::kWS + 256 * (wave % (TN / 64))), 4,
                                             (int)d.ws, ks_off, 0, 0);
}

// Per-wave operand state.  A stage's packed rows (16 code bytes and two E4M3
// scales per lane and row) are read from LDS once; each MFMA step ks widens its
// fragments from them (bf16 A fragments are read from LDS per step instead).
// Rows r0 + 32 i + l % 32 share the swizzle terms of l % 32, so every row's LDS
// offset is a per-lane base plus a constant.
template <int F, int L, int TM, int TN>
struct NvPipe {
    using S = NvTile<F == 1, L, TM, TN>;
    static constexpr int NA = F == kFmtNv44 ? S::NI : 1;
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    u32x4 wc[S::NJ];
    f32x2 wsc[S::NJ];  // W4A16: the lane's two block scales as fp32
    f16x2 wsh[S::NJ];  // W4A4: the same as fp16 (exact), for the fp16 widening
    u32x4 ac[NA];
    f16x2 ash[NA];
    uint32_t wb, wsb;  // W codes / scales of MFMA tile 0
    uint32_t ab, asb;  // A codes / scales (W4A4) or bf16 row (W4A16) of MFMA tile 0
    uint32_t ak[4];    // W4A16: swizzled 16-byte chunk of step ks in a bf16 A row
};

template <int F, int L, int TM, int TN>
__device__ __forceinline__ void nv_pipe_init(NvPipe<F, L, TM, TN> &p, int wave, int lane)
{
    using S = NvTile<F == 1, L, TM, TN>;
    const int half = lane >> 5, l = lane & 31;
    const int r0 = S::row0(wave), c0 = S::col0(wave);
    const int hsw = 16 * (half ^ ((l >> 3) & 1));
    p.wb = 32 * (c0 + l) + hsw;
    p.wsb = 4 * (c0 + l) + (F == kFmtMx16 ? half : 2 * half);
    if (F == kFmtNv44) {
        p.ab = 32 * (r0 + l) + hsw;
        p.asb = 4 * (r0 + l) + 2 * half;
    } else {
        p.ab = 128 * (r0 + l);
        p.asb = 0;
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) p.ak[ks] = 16 * ((4 * half + ks) ^ ((l >> 1) & 7));
}

// read the stage's packed rows (codes + scales) into registers
// (t: the stage's index; MXFP4 picks its E8M0 byte pair by t's parity).
// NIL: the wave's 32-row blocks that hold rows of the tile (the others are
// neither read nor multiplied; grouped tiles past their group's last row)
template <int F, int L, int TM, int TN, int NIL = NvTile<F == 1, L, TM, TN>::NI>
__device__ __forceinline__ void nv_pipe_raw(NvPipe<F, L, TM, TN> &p, const uint8_t *st, int t)
{
    using S = NvTile<F == 1, L, TM, TN>;
#pragma unroll
    for (int j = 0; j < S::NJ; ++j) {
        p.wc[j] = *reinterpret_cast<const u32x4 *>(st + S::kW + p.wb + 1024 * j);
        if constexpr (F == kFmtMx16) {
            // E8M0 byte e of the lane's 32-element block -> the fp32 2^(e - 127) the
            // scaled conversion takes its exponent from
            const uint32_t e = st[S::kWS + p.wsb + 2 * (t & 1) + 128 * j];
            p.wsc[j][0] = __uint_as_float(e << 23);
        } else if constexpr (F == kFmtNv44) {
            p.wsh[j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(
                (uint32_t)*reinterpret_cast<const uint16_t *>(st + S::kWS + p.wsb + 128 * j), 1.0f, false);
        } else {
            p.wsc[j] = __builtin_amdgcn_cvt_pk_f32_fp8(
                (int)*reinterpret_cast<const uint16_t *>(st + S::kWS + p.wsb + 128 * j), false);
        }
    }
    if constexpr (F == kFmtNv44) {
#pragma unroll
        for (int i = 0; i < NIL; ++i) {
            p.ac[i] = *reinterpret_cast<const u32x4 *>(st + S::kA + p.ab + 1024 * i);
            p.ash[i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(
                (uint32_t)*reinterpret_cast<const uint16_t *>(st + S::kAS + p.asb + 128 * i), 1.0f, false);
        }
    }
}

// fragments of step ks: lane half h holds K = 32 h + 8 ks + [0, 8) of the stage
template <int F, int L, int TM, int TN, int KS, int NIL = NvTile<F == 1, L, TM, TN>::NI>
__device__ __forceinline__ void nv_pipe_frags(const NvPipe<F, L, TM, TN> &p, const uint8_t *st,
                                              bf16x8 (&wf)[NvTile<F == 1, L, TM, TN>::NJ],
                                              bf16x8 (&af)[NvTile<F == 1, L, TM, TN>::NI])
{
    using S = NvTile<F == 1, L, TM, TN>;
#pragma unroll
    for (int j = 0; j < S::NJ; ++j) {
        if constexpr (F == kFmtMx16)
            wf[j] = e2m1x8_bf16_pow2(p.wc[j][KS], p.wsc[j][0]);
        else if constexpr (F == kFmtNv44)
            wf[j] = as_bf16x8(dq8_f16(p.wc[j][KS], KS < 2 ? p.wsh[j][0] : p.wsh[j][1]));
        else
            wf[j] = as_bf16x8(dq8_bf16(p.wc[j][KS], KS < 2 ? p.wsc[j][0] : p.wsc[j][1]));
    }
#pragma unroll
    for (int i = 0; i < NIL; ++i) {
        if constexpr (F == kFmtNv44)
            af[i] = as_bf16x8(dq8_f16(p.ac[i][KS], KS < 2 ? p.ash[i][0] : p.ash[i][1]));
        else
            af[i] = *reinterpret_cast<const bf16x8 *>(st + S::kA + p.ab + p.ak[KS] + 4096 * i);
    }
}

// F16: the fragments hold fp16 bits (W4A4, both operands widened exactly to fp16);
// row blocks NIL .. NI - 1 are left alone
template <int NI, int NJ, bool F16, int NIL = NI>
__device__ __forceinline__ void nv_pipe_mfma(f32x16 (&acc)[NI][NJ], const bf16x8 (&wf)[NJ], const bf16x8 (&af)[NI])
{
#pragma unroll
    for (int i = 0; i < NIL; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            if constexpr (F16)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, wf[j]),
                                                                   __builtin_bit_cast(f16x8, af[i]), acc[i][j], 0, 0, 0);
            else
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[j], af[i], acc[i][j], 0, 0, 0);
        }
}

// Spread the NM MFMAs of a step over the widening (NV VALU) and the reads (ND)
// of the next step.  NR reads go out first, then P MFMAs cover their latency
// before any VALU work uses them; the NB copies (global-to-LDS) are spread one per
// MFMA slot, since a burst of copies holds back the MFMAs behind it in the wave's
// instruction stream.
template <int N, int NV, int ND, int T, int NC = 0>
__device__ __forceinline__ void nv_pipe_slot()
{
    constexpr int v = NV * (T + 1) / N - NV * T / N, r = ND * (T + 1) / N - ND * T / N;
    constexpr int cp = NC * (T + 1) / N - NC * T / N;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    if constexpr (cp > 0) __builtin_amdgcn_sched_group_barrier(0x020, cp, 0);  // copies
    if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x002, v, 0);  // VALU
    if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);  // DS read
    if constexpr (T + 1 < N) nv_pipe_slot<N, NV, ND, T + 1, NC>();
}

template <int NM, int NV, int ND, int NR = 0, int NB = 0, int P = 0>
__device__ __forceinline__ void nv_pipe_interleave()
{
    if constexpr (NR > 0) __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);  // DS read
    if constexpr (P > 0) __builtin_amdgcn_sched_group_barrier(0x008, P, 0);    // MFMA
    nv_pipe_slot<NM - P, NV, ND, 0, NB>();
    __builtin_amdgcn_sched_barrier(0);
}

template <int N>
__device__ __forceinline__ void nv_wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One stage t (in `cur`; stage t + 1 in `nxt`).  Entering, wf / af hold step 0's
// fragments.  Steps 0-2 multiply while the next step's fragments are formed; then
// the wave waits until its copies of stage t + 1 landed and its reads of `cur`
// returned, and a barrier extends both to every wave, so `cur` is free: the copy
// of stage t + 3 starts into it.  Step 3 multiplies while stage t + 1's packed
// rows and step-0 fragments are read from `nxt`.  One basic block per stage.
template <int F, int L, int TM, int TN, int NIL = NvTile<F == 1, L, TM, TN>::NI>
__device__ __forceinline__ void nv_pipe_stage(uint8_t *cur, const uint8_t *nxt, int t, int nk, const NvRingDma &d,
                                              const NvRingDma &dz, int wave, NvPipe<F, L, TM, TN> &p,
                                              f32x16 (&acc)[NvTile<F == 1, L, TM, TN>::NI][NvTile<F == 1, L, TM, TN>::NJ],
                                              bf16x8 (&wf)[NvTile<F == 1, L, TM, TN>::NJ],
                                              bf16x8 (&af)[NvTile<F == 1, L, TM, TN>::NI])
{
    using S = NvTile<F == 1, L, TM, TN>;
    constexpr bool A_FP4 = F == kFmtNv44;
    constexpr int NI = S::NI, NJ = S::NJ, NM = NIL * NJ;
    static_assert(NIL >= 1 && NIL <= NI, "live row blocks");
    constexpr int NV = (F == kFmtMx16 ? 4 : A_FP4 ? 8 : 16) * (NJ + (A_FP4 ? NIL : 0));  // VALU per step's widening, about
    constexpr int ND = A_FP4 ? 0 : NIL;               // DS reads per step
    constexpr int P = NM >= 8 ? 4 : 1;
    bf16x8 wf1[NJ], af1[NI];
    nv_pipe_frags<F, L, TM, TN, 1, NIL>(p, cur, wf1, af1);
    nv_pipe_mfma<NI, NJ, A_FP4, NIL>(acc, wf, af);
    nv_pipe_interleave<NM, NV, ND>();
    nv_pipe_frags<F, L, TM, TN, 2, NIL>(p, cur, wf, af);
    nv_pipe_mfma<NI, NJ, A_FP4, NIL>(acc, wf1, af1);
    nv_pipe_interleave<NM, NV, ND>();
    nv_pipe_frags<F, L, TM, TN, 3, NIL>(p, cur, wf1, af1);
    nv_pipe_mfma<NI, NJ, A_FP4, NIL>(acc, wf, af);
    nv_pipe_interleave<NM, NV, ND>();
    nv_wait_vm<S::kDma>();
    __builtin_amdgcn_s_waitcnt((0xF) | (0x3 << 14) | (7 << 4));  // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
    nv_pipe_raw<F, L, TM, TN, NIL>(p, nxt, t + 1);
    nv_ring_dma<F, L, TM, TN>(cur, t + 3 < nk ? d : dz, (t + 3 < nk ? t + 3 : 0) * kRK, wave);
    nv_pipe_frags<F, L, TM, TN, 0, NIL>(p, nxt, wf, af);
    nv_pipe_mfma<NI, NJ, A_FP4, NIL>(acc, wf1, af1);
    nv_pipe_interleave<NM, NV, ND, 2 * (A_FP4 ? NIL + NJ : NJ), S::kDma, P>();
}

// The K loop of a tile: the first stage's fragments, then the stages in threes
// (the three LDS stages rotate), then the last one or two (no copies left to
// start).  Every variant runs the same copies and barriers, so waves of one
// workgroup may take different NIL.
template <int F, int L, int TM, int TN, int NIL>
__device__ __forceinline__ void nv_ring_kloop(uint8_t *s0, uint8_t *s1, uint8_t *s2, int nk, const NvRingDma &d,
                                              const NvRingDma &dz, int wave, NvPipe<F, L, TM, TN> &p,
                                              f32x16 (&acc)[NvTile<F == 1, L, TM, TN>::NI][NvTile<F == 1, L, TM, TN>::NJ])
{
    using S = NvTile<F == 1, L, TM, TN>;
    bf16x8 wf[S::NJ], af[S::NI];
    nv_pipe_raw<F, L, TM, TN, NIL>(p, s0, 0);
    nv_pipe_frags<F, L, TM, TN, 0, NIL>(p, s0, wf, af);
    const int nfull = nk - nk % 3;
    for (int t = 0; t < nfull; t += 3) {
        nv_pipe_stage<F, L, TM, TN, NIL>(s0, s1, t, nk, d, dz, wave, p, acc, wf, af);
        nv_pipe_stage<F, L, TM, TN, NIL>(s1, s2, t + 1, nk, d, dz, wave, p, acc, wf, af);
        nv_pipe_stage<F, L, TM, TN, NIL>(s2, s0, t + 2, nk, d, dz, wave, p, acc, wf, af);
    }
    if (nk % 3 >= 1) nv_pipe_stage<F, L, TM, TN, NIL>(s0, s1, nfull, nk, d, dz, wave, p, acc, wf, af);
    if (nk % 3 == 2) nv_pipe_stage<F, L, TM, TN, NIL>(s1, s2, nfull + 1, nk, d, dz, wave, p, acc, wf, af);
}

// Epilogue: lane l holds output row r0 + 32 i + l % 32, columns
// c0 + 32 j + 8 g + 4 (l / 32) + 0..3 in slots 4 g .. 4 g + 3 of acc[i][j].  In
// round rd, tile rows rd R + [0, R) go through `s0` and rows H + rd R + [0, R)
// through `s1` (H = TM / 2), then leave as whole-row 16-byte stores.
template <typename T, int F, int L, int TM, int TN>
__device__ __forceinline__ void nv_ring_epilogue(
    const f32x16 (&acc)[NvTile<F == 1, L, TM, TN>::NI][NvTile<F == 1, L, TM, TN>::NJ], uint8_t *s0, uint8_t *s1,
    const NvGemmArgs &g, int m0, int n0, int wave, int lane, int tid, const int32_t *ridx = nullptr,
    int a_rows = 0)
{
    using S = NvTile<F == 1, L, TM, TN>;
    constexpr int NI = S::NI, NJ = S::NJ, H = S::H;
    constexpr int es = (int)sizeof(T);
    constexpr int pitch = S::epi_pitch(es);
    constexpr int R = S::epi_rows(es);
    constexpr int kPer = 16 / es, kChunks = TN / kPer;
    static_assert(R * pitch <= S::stage_bytes(es), "epilogue staging");
    constexpr bool A_FP4 = F == kFmtNv44;
    const int M = (int)g.M, N = (int)g.N;
    const float wt = F == kFmtMx16 ? 1.f : g.w_tscale[0];  // MXFP4 has no tensor scale
    const int r0 = S::row0(wave), c0 = S::col0(wave);
#pragma unroll
    for (int rd = 0; rd < H / R; ++rd) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            // rows of MFMA tile i: r0 + 32 i + [0, 32), one staging buffer, one round
            const int rr = L ? (32 * i) % H : 32 * i;  // row within its half of the tile
            if (rr / R != rd) continue;
            const int m = m0 + r0 + 32 * i + (lane & 31);
            float sc = wt;
            if (A_FP4) {
                int am = m < M ? m : -1;  // the row's A row, for its per-row scale
                if (ridx && am >= 0) am = (uint32_t)ridx[m] < (uint32_t)a_rows ? ridx[m] : -1;
                sc = (am >= 0 ? g.a_tscale[g.a_per_row ? am : 0] : 0.f) * wt;
            }
            uint8_t *buf = (L ? 32 * i : r0) >= H ? s1 : s0;
            uint8_t *row = buf + (rr - rd * R + (lane & 31)) * pitch;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const int col = c0 + 32 * j + 8 * gq + 4 * (lane >> 5);
                    const f32x16 &a = acc[i][j];
                    if constexpr (es == 2) {
                        const bf16x4 v = {(__bf16)(a[4 * gq] * sc), (__bf16)(a[4 * gq + 1] * sc),
                                          (__bf16)(a[4 * gq + 2] * sc), (__bf16)(a[4 * gq + 3] * sc)};
                        *reinterpret_cast<bf16x4 *>(row + 2 * col) = v;
                    } else {
                        *reinterpret_cast<f32x4 *>(row + 4 * col) =
                            f32x4{a[4 * gq] * sc, a[4 * gq + 1] * sc, a[4 * gq + 2] * sc, a[4 * gq + 3] * sc};
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        __syncthreads();
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const uint8_t *st = half ? s1 : s0;
            const int mrow0 = m0 + H * half + rd * R;
            for (int q = tid; q < R * kChunks; q += 256) {
                const int r = q / kChunks, ch = q % kChunks;
                const int m = mrow0 + r, n = n0 + ch * kPer;
                if (m >= M || n >= N) continue;
                const uint4 v = *reinterpret_cast<const uint4 *>(st + r * pitch + 16 * ch);
                T *dstp = reinterpret_cast<T *>(g.c) + (int64_t)m * g.ldc + n;
                if (n + kPer <= N) {
                    *reinterpret_cast<uint4 *>(dstp) = v;
                } else {
                    T e[kPer];
                    __builtin_memcpy(e, &v, 16);
#pragma unroll
                    for (int tt = 0; tt < kPer; ++tt)
                        if (n + tt < N) dstp[tt] = e[tt];
                }
            }
        }
        __syncthreads();
    }
}

__device__ __forceinline__ int nv_wave_incl_scan(int v, int lane)
{
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int t = __shfl_up(v, d);
        if (lane >= d) v += t;
    }
    return v;
}

// Grouped (MoE) launches.  Group e owns grouped rows [offs[e], offs[e + 1])
// (each clamped to [0, M]) and needs ceil(rows / TM) * tiles_n tiles.  Every
// wave scans the offsets 64 groups at a time: the total tile count first (blocks
// at or past it leave), then the group that holds this block's tile.  Block b
// takes logical tile L in the XCD-aware order of tile_of; within a group the tile
// rows vary fastest, so the tiles that share a weight panel sit together.
template <int TM, int TN>
__device__ __forceinline__ bool nv_group_tile(const NvGemmArgs &g, int b, int &e, int &tm, int &tn, int &row0,
                                              int &rows)
{
    const int T = (int)g.M, E = g.groups, tiles_n = ((int)g.N + TN - 1) / TN;
    const int lane = threadIdx.x & 63, passes = (E + 63) / 64;
    auto group = [&](int c, int &lo, int &hi) -> int {  // tiles of group 64 c + lane
        const int i = 64 * c + lane;
        lo = hi = 0;
        if (i >= E) return 0;
        lo = min(max(g.group_offs[i], 0), T);
        hi = min(max(g.group_offs[i + 1], 0), T);
        return hi > lo ? ((hi - lo + TM - 1) / TM) * tiles_n : 0;
    };
    int total = 0;
    for (int c = 0; c < passes; ++c) {
        int lo, hi;
        total += __shfl(nv_wave_incl_scan(group(c, lo, hi), lane), 63);
    }
    total = __builtin_amdgcn_readfirstlane(total);
    if (b >= total) return false;
    const int per = (total + 7) / 8, xcd = b % 8, idx = b / 8, full = total % 8;
    const int L = full == 0 || xcd < full ? xcd * per + idx : full * per + (xcd - full) * (per - 1) + idx;
    int before = 0;
    for (int c = 0; c < passes; ++c) {
        int lo, hi;
        const int n = group(c, lo, hi);
        const int incl = nv_wave_incl_scan(n, lane);
        const int sum = __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
        if (L < before + sum) {
            const int j = (int)__builtin_ctzll(__ballot(before + incl > L));
            e = 64 * c + j;
            const int start = before + __builtin_amdgcn_readfirstlane(__shfl(incl - n, j));
            row0 = __builtin_amdgcn_readfirstlane(__shfl(lo, j));
            rows = __builtin_amdgcn_readfirstlane(__shfl(hi, j)) - row0;
            const int tiles_me = (rows + TM - 1) / TM, li = L - start;
            tm = li % tiles_me;
            tn = li / tiles_me;
            return true;
        }
        before += sum;
    }
    return false;
}

// GR: the grouped form (one weight per group, rows by group offsets, optional
// row gather from A; see NvGemmArgs)
template <int F, int L, typename OutT, int TM, int TN, bool GR = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(TM == 128 && TN == 256 ? 2 : 1)))
void k_nv_gemm_ring(NvGemmArgs g)
{
    using S = NvTile<F == 1, L, TM, TN>;
    constexpr bool A_FP4 = F == kFmtNv44;
    constexpr int kWsRow = F == kFmtMx16 ? 32 : 16;  // K elements per weight scale byte
    constexpr int NI = S::NI, NJ = S::NJ;
    constexpr int kStage = S::stage_bytes((int)sizeof(OutT));
    __shared__ __align__(16) uint8_t s0[kStage];
    __shared__ __align__(16) uint8_t s1[kStage];
    __shared__ __align__(16) uint8_t s2[kStage];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int N = (int)g.N, K = (int)g.K;
    const int tiles_n = (N + TN - 1) / TN;
    int tm, tn;
    const int32_t *ridx = nullptr;  // grouped row -> A row (gathered groups)
    int a_rows = (int)g.M;          // rows the A descriptors cover
    if constexpr (GR) {
        int e, row0, rows;
        if (!nv_group_tile<TM, TN>(g, blockIdx.x, e, tm, tn, row0, rows)) return;
        g.w_codes += (int64_t)e * N * (K / 2);
        g.w_scales += (int64_t)e * N * (K / kWsRow);
        if constexpr (F != kFmtMx16) g.w_tscale += e;
        g.c = reinterpret_cast<uint8_t *>(g.c) + (int64_t)row0 * g.ldc * (int64_t)sizeof(OutT);
        g.M = rows;
        if (g.row_index) {
            ridx = g.row_index + row0;
            a_rows = (int)g.a_rows;
        } else {
            a_rows = rows;
            if constexpr (A_FP4) {
                g.a_codes += (int64_t)row0 * (K / 2);
                g.a_scales += (int64_t)row0 * (K / 16);
                if (g.a_per_row) g.a_tscale += row0;
            } else {
                g.a += (int64_t)row0 * g.lda;
            }
        }
    } else {
        tile_of(blockIdx.x, gridDim.x, ((int)g.M + TM - 1) / TM, tiles_n, tm, tn);
    }
    const int M = (int)g.M;
    const int m0 = tm * TM, n0 = tn * TN;
    const int nk = K / kRK;
    // A row of tile row m (-1: none; a gathered index outside A counts as none)
    auto arow = [&](int m) -> int {
        if (m >= M) return -1;
        if constexpr (GR) {
            if (ridx) {
                const int v = ridx[m];
                return (uint32_t)v < (uint32_t)a_rows ? v : -1;
            }
        }
        return m;
    };

    NvRingDma d, dz;
    const int64_t w_rows = g.w_seg ? g.w_rows : N;  // rows the W descriptors cover
    d.rw = nv_rsrc(g.w_codes, w_rows * (K / 2));
    d.rws = nv_rsrc(g.w_scales, w_rows * (K / kWsRow));
    d.seg = g.w_seg;
    d.seg_w = (uint32_t)w_rows * 64u;
    d.seg_s = (uint32_t)w_rows * (F == kFmtMx16 ? 4u : 8u);
    if constexpr (A_FP4) {
        d.ra = nv_rsrc(g.a_codes, (int64_t)a_rows * (K / 2));
        d.ras = nv_rsrc(g.a_scales, (int64_t)a_rows * (K / 16));
#pragma unroll
        for (int i = 0; i < S::nA; ++i) {
            const int q = 64 * S::nA * wave + 64 * i + lane;
            const int r = q >> 1, h = (q & 1) ^ ((r >> 3) & 1);
            const int ar = arow(m0 + r);
            d.a[i] = ar >= 0 ? (uint32_t)ar * (uint32_t)(K / 2) + 16 * h : kNvOut;
        }
        const int qa = (64 * wave + lane) % TM;
        const int ara = arow(m0 + qa);
        d.as = ara >= 0 ? (uint32_t)ara * (uint32_t)(K / 16) : kNvOut;
    } else {
        d.ra = nv_rsrc(g.a, ((int64_t)(a_rows - 1) * g.lda + K) * 2);
        d.ras = d.ra;
#pragma unroll
        for (int i = 0; i < S::nA; ++i) {
            const int q = 64 * S::nA * wave + 64 * i + lane;
            const int r = q >> 3, c = (q & 7) ^ ((r >> 1) & 7);
            const int ar = arow(m0 + r);
            d.a[i] = ar >= 0 ? (uint32_t)(((int64_t)ar * g.lda + 8 * c) * 2) : kNvOut;
        }
        d.as = kNvOut;
    }
#pragma unroll
    for (int i = 0; i < S::nW; ++i) {
        const int q = 64 * S::nW * wave + 64 * i + lane;
        const int r = q >> 1, h = (q & 1) ^ ((r >> 3) & 1);
        const uint32_t wr = g.w_seg ? (uint32_t)(g.w_row0 + n0 + r) * 64u : (uint32_t)(n0 + r) * (uint32_t)(K / 2);
        d.w[i] = n0 + r < N ? wr + 16 * h : kNvOut;
    }
    const int qw = (64 * wave + lane) % TN;
    const uint32_t wsr = g.w_seg ? (uint32_t)(g.w_row0 + n0 + qw) * (F == kFmtMx16 ? 4u : 8u)
                                 : (uint32_t)(n0 + qw) * (uint32_t)(K / kWsRow);
    d.ws = n0 + qw < N ? wsr : kNvOut;
    dz = d;
    dz.ra = nv_rsrc(g.a_codes ? (const void *)g.a_codes : (const void *)g.a, 0);
    dz.ras = dz.ra;
    dz.rw = nv_rsrc(g.w_codes, 0);
    dz.rws = nv_rsrc(g.w_scales, 0);

    f32x16 acc[NI][NJ];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{};

    NvPipe<F, L, TM, TN> p;
    nv_pipe_init(p, wave, lane);
    nv_ring_dma<F, L, TM, TN>(s0, d, 0, wave);
    nv_ring_dma<F, L, TM, TN>(s1, nk > 1 ? d : dz, nk > 1 ? kRK : 0, wave);
    nv_ring_dma<F, L, TM, TN>(s2, nk > 2 ? d : dz, nk > 2 ? 2 * kRK : 0, wave);
    nv_wait_vm<2 * S::kDma>();
    asm volatile("s_barrier" ::: "memory");
    // A grouped 128-row tile multiplies only the 32-row blocks that hold rows of
    // its group (the group's last tile is on average half empty): each wave
    // picks the K loop for its live blocks
    if constexpr (GR && TM == 128) {
        const int live = min(TM, M - m0) - S::row0(wave);  // rows of this wave's blocks
        const int nil = min(NI, max(1, (live + 31) / 32));
        if (nil == 1) nv_ring_kloop<F, L, TM, TN, 1>(s0, s1, s2, nk, d, dz, wave, p, acc);
        else if constexpr (NI > 2) {
            if (nil == 2) nv_ring_kloop<F, L, TM, TN, 2>(s0, s1, s2, nk, d, dz, wave, p, acc);
            else if (nil == 3) nv_ring_kloop<F, L, TM, TN, 3>(s0, s1, s2, nk, d, dz, wave, p, acc);
            else nv_ring_kloop<F, L, TM, TN, NI>(s0, s1, s2, nk, d, dz, wave, p, acc);
        } else {
            nv_ring_kloop<F, L, TM, TN, NI>(s0, s1, s2, nk, d, dz, wave, p, acc);
        }
    } else {
        nv_ring_kloop<F, L, TM, TN, NI>(s0, s1, s2, nk, d, dz, wave, p, acc);
    }
    __builtin_amdgcn_s_waitcnt(0);  // the last (empty) copies landed
    __syncthreads();
    const int lane_e = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    nv_ring_epilogue<OutT, F, L, TM, TN>(acc, s0, s1, g, m0, n0, wave, lane_e, 64 * wave + lane_e, ridx, a_rows);
}

constexpr size_t kGemmLds = (size_t)2 * (BM + BN) * BK * sizeof(uint16_t);  // 128 KiB

template <bool A_FP4, bool ALIGNED>
static fp4_status launch_prefill(const NvGemmArgs &g, hipStream_t st)
{
    static std::atomic<uint64_t> lds_set{0};  // per device
    if (!set_max_lds_once((const void *)k_nv_gemm<A_FP4, ALIGNED>, (int)kGemmLds, lds_set)) return FP4_ERR_HIP;
    const int tiles = (int)(((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN));
    hipLaunchKernelGGL((k_nv_gemm<A_FP4, ALIGNED>), dim3(tiles), dim3(256), kGemmLds, st, g);
    return hipGetLastError() == hipSuccess ? FP4_OK : FP4_ERR_HIP;
}

template <int F, int L, int TM, int TN>
static void launch_ring(const NvGemmArgs &g, hipStream_t st)
{
    const int tiles = (int)(((g.M + TM - 1) / TM) * ((g.N + TN - 1) / TN));
    if (g.c_bf16)
        hipLaunchKernelGGL((k_nv_gemm_ring<F, L, __bf16, TM, TN>), dim3(tiles), dim3(256), 0, st, g);
    else
        hipLaunchKernelGGL((k_nv_gemm_ring<F, L, float, TM, TN>), dim3(tiles), dim3(256), 0, st, g);
}

// 256 x 256 tiles; when the last round of tiles would leave most CUs idle, the
// tile columns of that round go to a second launch of 128 x 128 tiles, provided
// they fit in one round (for M = 4096, N = 17408: 1024 large tiles, four full
// rounds on 256 CUs, then 256 small tiles for the last 1024 columns), else of
// 128 x 256 tiles if those fit (M = 8192: eight full rounds, then 256 tiles of
// 128 x 256 where a ninth round of 128 large tiles left half the CUs idle).
template <int F, int L>
static void launch_ring_split(const NvGemmArgs &g, hipStream_t st)
{
    const int64_t cus = device_cu_count();
    const int64_t tm = (g.M + 255) / 256, tn = (g.N + 255) / 256, tiles = tm * tn;
    const int64_t rem = tiles % cus;
    if (tiles > cus && rem != 0 && rem <= cus / 2) {
        const int64_t cols = tiles / cus * cus / tm;  // 256-wide column blocks kept on large tiles
        const int64_t n_split = cols * 256;
        const int64_t small = ((g.M + 127) / 128) * ((g.N - n_split + 127) / 128);
        const int64_t mid = ((g.M + 127) / 128) * ((g.N - n_split + 255) / 256);
        if (cols >= 1 && n_split < g.N && (small <= cus || mid <= cus)) {
            NvGemmArgs big = g;
            big.N = n_split;
            launch_ring<F, L, 256, 256>(big, st);
            NvGemmArgs rest = g;
            rest.N = g.N - n_split;
            if (g.w_seg) {
                rest.w_row0 = g.w_row0 + n_split;  // the decode layout interleaves rows per segment
            } else {
                rest.w_codes = g.w_codes + n_split * (g.K / 2);
                rest.w_scales = g.w_scales + n_split * (g.K / (F == kFmtMx16 ? 32 : 16));
            }
            rest.c = reinterpret_cast<uint8_t *>(g.c) + n_split * (g.c_bf16 ? 2 : 4);
            if (small <= cus)
                launch_ring<F, L, 128, 128>(rest, st);  // W4A16: each wave 128 rows x 32 columns
            else
                launch_ring<F, L, 128, 256>(rest, st);  // M = 8192, N = 17408: 256 tiles of 128 x 256
            return;
        }
    }
    launch_ring<F, L, 256, 256>(g, st);
}

// Grouped launches: the grid is an upper bound of the tile count (sum over groups
// of ceil(rows / TM) <= ceil(M / TM) + groups); blocks past the real count leave
// at once.  TM = 128 unless groups average 512 rows or more (the last tile of a
// group is on average half empty).
template <int F, int L, int TM>
static void launch_ring_grouped(const NvGemmArgs &g, hipStream_t st)
{
    const int64_t grid = ((g.M + TM - 1) / TM + g.groups) * ((g.N + 255) / 256);
    if (g.c_bf16)
        hipLaunchKernelGGL((k_nv_gemm_ring<F, L, __bf16, TM, 256, true>), dim3((unsigned)grid), dim3(256), 0, st, g);
    else
        hipLaunchKernelGGL((k_nv_gemm_ring<F, L, float, TM, 256, true>), dim3((unsigned)grid), dim3(256), 0, st, g);
}

fp4_status launch_grouped_gemm(const NvGemmArgs &g, int fmt, hipStream_t st)
{
    const bool a_fp4 = fmt == kFmtNv44;
    // 32-bit byte offsets into A and into one group's weight
    const int64_t a_bytes = a_fp4 ? g.a_rows * (g.K / 2) : g.a_rows * g.lda * 2;
    if (g.K % (fmt == kFmtMx16 ? 128 : kRK) != 0 || a_bytes >= (int64_t(1) << 31) ||
        g.N * (g.K / 2) >= (int64_t(1) << 31))
        return FP4_ERR_SHAPE;
    if (((g.M + 127) / 128 + g.groups) * ((g.N + 255) / 256) >= (int64_t(1) << 31)) return FP4_ERR_SHAPE;
    const bool big = g.M >= 512 * (int64_t)g.groups;
    switch (fmt) {
    case kFmtNv16:
        big ? launch_ring_grouped<kFmtNv16, kNvL16, 256>(g, st) : launch_ring_grouped<kFmtNv16, kNvL16, 128>(g, st);
        break;
    case kFmtNv44:
        big ? launch_ring_grouped<kFmtNv44, 0, 256>(g, st) : launch_ring_grouped<kFmtNv44, 0, 128>(g, st);
        break;
    default:
        big ? launch_ring_grouped<kFmtMx16, kNvL16, 256>(g, st) : launch_ring_grouped<kFmtMx16, kNvL16, 128>(g, st);
        break;
    }
    return hipGetLastError() == hipSuccess ? FP4_OK : FP4_ERR_HIP;
}

fp4_status launch_gemm_w4a16_seg(const NvGemmArgs &g, bool mx, hipStream_t st)
{
    // the ring kernel addresses operands with 32-bit byte offsets
    if (g.K % 128 != 0 || g.M * g.lda * 2 >= (int64_t(1) << 31) || g.w_rows * (g.K / 2) >= (int64_t(1) << 31))
        return FP4_ERR_SHAPE;
    if (mx) launch_ring_split<kFmtMx16, kNvL16>(g, st);
    else launch_ring_split<kFmtNv16, kNvL16>(g, st);
    return hipGetLastError() == hipSuccess ? FP4_OK : FP4_ERR_HIP;
}

fp4_status launch_gemm_w4a4_seg(const NvGemmArgs &g, hipStream_t st)
{
    // the ring kernel addresses operands with 32-bit byte offsets
    if (g.K % 128 != 0 || g.M * (g.K / 2) >= (int64_t(1) << 31) || g.w_rows * (g.K / 2) >= (int64_t(1) << 31))
        return FP4_ERR_SHAPE;
    launch_ring_split<kFmtNv44, 0>(g, st);
    return hipGetLastError() == hipSuccess ? FP4_OK : FP4_ERR_HIP;
}

fp4_status launch_mxfp4_gemm_w4a16(const NvGemmArgs &g, hipStream_t st)
{
    // the ring kernel addresses operands with 32-bit byte offsets
    if (g.K % 128 != 0 || g.M * g.lda * 2 >= (int64_t(1) << 31) || g.N * (g.K / 2) >= (int64_t(1) << 31))
        return FP4_ERR_SHAPE;
    launch_ring_split<kFmtMx16, kNvL16>(g, st);
    return hipGetLastError() == hipSuccess ? FP4_OK : FP4_ERR_HIP;
}

fp4_status launch_nvfp4_gemm(const NvGemmArgs &g, hipStream_t st)
{
    const bool aligned = (g.K % 64) == 0;
    if (!g.a_codes && g.M <= 16) {
        if (g.K % 1024 == 0 && g.K <= 8192) {
            switch (g.K / 1024) {
            case 1: return launch_decode_persist<1>(g, st);
            case 2: return launch_decode_persist<2>(g, st);
            case 3: return launch_decode_persist<3>(g, st);
            case 4: return launch_decode_persist<4>(g, st);
            case 5: return launch_decode_persist<5>(g, st);
            case 6: return launch_decode_persist<6>(g, st);
            case 7: return launch_decode_persist<7>(g, st);
            default: return launch_decode_persist<8>(g, st);
            }
        }
        if (g.K % 128 == 0) {
            hipLaunchKernelGGL(k_nv_decode, dim3((unsigned)((g.N + 15) / 16)), dim3(256), 0, st, g.a, g.lda,
                               g.w_codes, g.w_scales, g.w_tscale, (int)g.M, (int)g.N, (int)g.K, g.c,
                               g.c_bf16, g.ldc);
            return hipGetLastError() == hipSuccess ? FP4_OK : FP4_ERR_HIP;
        }
        const int nwg = (int)((g.N + 16 * kDecNT - 1) / (16 * kDecNT));
        if (aligned)
            hipLaunchKernelGGL(k_nv_decode_generic<true>, dim3(nwg), dim3(64 * kDecWaves), 0, st, g.a,
                               g.lda, g.w_codes, g.w_scales, g.w_tscale, (int)g.M, (int)g.N, (int)g.K,
                               g.c, g.c_bf16, g.ldc);
        else
            hipLaunchKernelGGL(k_nv_decode_generic<false>, dim3(nwg), dim3(64 * kDecWaves), 0, st, g.a,
                               g.lda, g.w_codes, g.w_scales, g.w_tscale, (int)g.M, (int)g.N, (int)g.K,
                               g.c, g.c_bf16, g.ldc);
        return hipGetLastError() == hipSuccess ? FP4_OK : FP4_ERR_HIP;
    }
    // the ring kernel addresses operands with 32-bit byte offsets
    const bool ring = aligned && g.M * g.K * 2 < (int64_t(1) << 31) && g.N * (g.K / 2) < (int64_t(1) << 31) &&
                      (g.a_codes || g.M * g.lda * 2 < (int64_t(1) << 31));
    if (ring) {
        if (g.a_codes) launch_ring_split<1, 0>(g, st);
        else launch_ring_split<0, kNvL16>(g, st);
        return hipGetLastError() == hipSuccess ? FP4_OK : FP4_ERR_HIP;
    }
    if (g.a_codes)
        return aligned ? launch_prefill<true, true>(g, st) : launch_prefill<true, false>(g, st);
    return aligned ? launch_prefill<false, true>(g, st) : launch_prefill<false, false>(g, st);
}

}  // namespace fp4k
