// gemm_mx.hip -- MXFP4 W4A4 GEMM on gfx950's block-scaled FP4 matrix instruction.
//
// MXFP4 (edge-FP4 article, eefocus.com, section "FP4 as the next core
// standard"): OCP MX block floating point, 32 contiguous K-elements share one
// E8M0 (power-of-two) scale, elements E2M1.  v_mfma_scale_f32_32x32x64_f8f6f4
// with both operand formats set to FP4 takes exactly that: each lane supplies 32
// FP4 values (16 bytes, low nibble first) of one row and that row's E8M0 byte
// for those 32 K-elements.  Products of two E2M1 values times two powers of two
// are exact; the matrix core accumulates in fp32.
//
// Tiling: 256 x 256 output tile per workgroup.  Packed codes and scale bytes are
// staged in LDS unchanged.  K % 256 == 0 takes the staged kernel (8 waves of
// 128 x 64, two 256-element LDS stages filled by global-to-LDS DMA); other K
// take a register-prefetch kernel (4 waves of 128 x 128) with 128-element steps
// that masks the K tail.
#include "device_common.h"
#include "internal.h"

namespace fp4k {

typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int MBM = 256, MBN = 256, MBK = 128;        // MBK: K elements per step of the prefetch kernel
constexpr int kRowBytes = MBK / 2;                    // 64 code bytes per row per step
constexpr int kMxGroupM = 8;

typedef __attribute__((address_space(3))) void mx_lds_void;

// LDS slot (16-byte units) of code chunk c (0..3) of tile row r: the chunk index is
// XORed with bits 2..3 of the row so that the 16 lanes of an MFMA fragment read
// (16 consecutive rows, one chunk) hit 16 different bank groups.
__device__ __forceinline__ int mswz(int row, int chunk) { return row * kRowBytes + ((chunk ^ ((row >> 2) & 3)) << 4); }


__device__ __forceinline__ void mx_tile_of(int b, int nb, int tiles_m, int tiles_n, int &tm, int &tn)
{
    const int per = (nb + 7) / 8;
    const int xcd = b % 8, idx = b / 8;
    const int full = nb % 8;
    const int logical = (full == 0 || xcd < full) ? xcd * per + idx
                                                  : full * per + (xcd - full) * (per - 1) + idx;
    const int group = logical / (kMxGroupM * tiles_n);
    const int first_m = group * kMxGroupM;
    const int gsz = min(kMxGroupM, tiles_m - first_m);
    const int in = logical % (kMxGroupM * tiles_n);
    tm = first_m + in % gsz;
    tn = in / gsz;
}

// Epilogue of the MX GEMM: each wave's 128 x 128 fp32 block (4 x 4 tiles of
// 32 x 32, accumulator slot e of tile (i, j) = row 32 i + 8 (e / 4) + 4 (lane / 32)
// + e % 4, column 32 j + lane % 32) is converted and staged through LDS 64 rows at
// a time (row stride padded by 16 bytes), then written with 16-byte
// row-contiguous stores.  `stage` holds 64 x (128 * 4 + 16) bytes for this wave.
constexpr int kMxStageRows = 64;
constexpr int kMxStagePitch = 128 * 4 + 16;

__device__ __forceinline__ void mx_store_block(const f32x16 (&acc)[4][4], uint8_t *stage, void *c,
                                               int c_bf16, int64_t ldc, int64_t r0, int64_t c0,
                                               int64_t M, int64_t N, int lane)
{
    const int es = c_bf16 ? 2 : 4;
    const int cpr = 128 * es / 16;  // 16-byte chunks per row
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int r = 32 * ii + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                    const int col = 32 * j + (lane & 31);
                    const float v = acc[2 * h + ii][j][e];
                    if (c_bf16)
                        *reinterpret_cast<uint16_t *>(stage + r * kMxStagePitch + 2 * col) = (uint16_t)f32_to_bf16_rne(v);
                    else
                        *reinterpret_cast<float *>(stage + r * kMxStagePitch + 4 * col) = v;
                }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        for (int q = lane; q < kMxStageRows * cpr; q += 64) {
            const int r = q / cpr, ch = q % cpr;
            const int64_t m = r0 + 64 * h + r, n = c0 + ch * (16 / es);
            if (m >= M) continue;
            const uint4 v = *reinterpret_cast<const uint4 *>(stage + r * kMxStagePitch + ch * 16);
            uint8_t *dst = reinterpret_cast<uint8_t *>(c) + (m * ldc + n) * es;
            if (n + 16 / es <= N && ((reinterpret_cast<uintptr_t>(dst) & 15) == 0)) {
                *reinterpret_cast<uint4 *>(dst) = v;
            } else {
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
                for (int t = 0; t < 16 / es; ++t) {
                    if (n + t >= N) break;
                    if (es == 2) reinterpret_cast<uint16_t *>(dst)[t] = (uint16_t)(w[t >> 1] >> (16 * (t & 1)));
                    else reinterpret_cast<uint32_t *>(dst)[t] = w[t];
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

// ---- main path (K % 256 == 0): two LDS stages of 256 K-elements fed by DMA ----
//
// 8 waves, two per SIMD, as 2 (M) x 4 (N) blocks of 128 x 64 outputs (4 x 2 MFMA
// tiles of 32 x 32): while one wave of a SIMD waits on LDS or the barrier the
// other keeps the matrix core busy, and 8 waves read LDS at almost twice the rate
// 4 waves reach.  Each stage holds, for both operands, 256 tile rows x 128 code bytes (16-byte
// chunk c of row r at slot 8 r + (c ^ ((r >> 1) & 7)), so the 16 lanes of an MFMA
// fragment read hit 16 different bank groups) and 256 rows x 8 E8M0 bytes.  The
// two stages are separate LDS objects: the compiler can then tell a DMA into one
// from a read of the other and does not wait for the DMA before the read.  Stage
// kt + 1 is copied while stage kt is multiplied; the barrier that publishes it
// sits in the middle of the last 64-element step of stage kt, and the fragments of
// the next step are read while the MFMAs of the current one run.
constexpr int kSK = 256;                          // K elements per stage
constexpr int kSRow = kSK / 2;                    // 128 code bytes per tile row
constexpr int kSTile = MBM * kSRow;               // 32 KiB of codes per operand
constexpr int kSScl = MBM * (kSK / 32);           // 2 KiB of scale bytes per operand
constexpr int kSStage = 2 * kSTile + 2 * kSScl;   // 69,632 bytes
static_assert(2 * kMxStageRows * kMxStagePitch <= kSStage, "two waves' output staging must fit a stage");

// Per-lane byte offsets (from the matrix base at k0 = 0) of the 10 DMA transfers a
// wave issues per stage: 4 x 16 bytes of A codes, 4 of W codes, one 4-byte scale
// dword per operand.  Code slot q = 256 wave + 64 i + lane is row q / 8, chunk
// (q % 8) ^ ((row >> 1) & 7); scale dword q = 64 wave + lane is row q / 2, bytes
// 4 (q % 2) .. +3.  Rows past the matrix edge re-read the last row: their
// products land only in outputs that are never stored.  The copies are buffer
// loads into LDS: a 32-bit per-lane offset, the stage's K offset as the scalar
// offset, and a descriptor per matrix whose size bound makes the hardware return
// zeros for any address past the matrix.  A stage that does not exist is
// "copied" through descriptors of size 0: the hardware writes zeros and reads
// nothing, so every stage runs the same code.
struct Mx2Dma {
    __amdgpu_buffer_rsrc_t ra, rw, rsa, rsw;
    uint32_t a[4], w[4], as, ws;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t mx2_rsrc(const uint8_t *base, int64_t bytes)
{
    // dword 3: data format 32 bits (a raw byte-addressed buffer; stride 0)
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(base), (short)0, (int)(uint32_t)bytes, 0x00020000);
}

__device__ __forceinline__ void mx2_dma(uint8_t *st, const Mx2Dma &d, int k0, int wave)
{
    // d's descriptors are chosen by the caller (matrix or empty)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(d.ra, (mx_lds_void *)(st + 16 * (256 * wave + 64 * i)), 16,
                                                 (int)d.a[i], k0 / 2, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rw, (mx_lds_void *)(st + kSTile + 16 * (256 * wave + 64 * i)), 16,
                                                 (int)d.w[i], k0 / 2, 0, 0);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rsa, (mx_lds_void *)(st + 2 * kSTile + 4 * (64 * wave)), 4, (int)d.as,
                                             k0 / 32, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rsw, (mx_lds_void *)(st + 2 * kSTile + kSScl + 4 * (64 * wave)), 4,
                                             (int)d.ws, k0 / 32, 0, 0);
}

// LDS offsets one lane reads within a stage: fragment (i, ks) of A is at
// la[ks] + 4096 i (i < 4), of W at lw[ks] + 4096 j (j < 2); the 8 scale bytes of
// A row i at lsa + 256 i, of W row j at lsw + 256 j.
struct Mx2Lds {
    uint32_t la[4], lw[4], lsa, lsw, sel;
};

struct Mx2Frag {
    i32x4 a[4], w[2];
};

__device__ __forceinline__ void mx2_frags(const uint8_t *st, uint32_t la, uint32_t lw, Mx2Frag &f)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) f.a[i] = *reinterpret_cast<const i32x4 *>(st + la + 4096 * i);
#pragma unroll
    for (int j = 0; j < 2; ++j) f.w[j] = *reinterpret_cast<const i32x4 *>(st + lw + 4096 * j);
}

// The lane's MFMA scale operand for step ks is byte ks of one dword: lanes 0..31
// supply blocks 0, 2, 4, 6 of the row's 8 blocks in the stage, lanes 32..63
// blocks 1, 3, 5, 7 (the K-half of the 32 x 32 x 64 instruction each half covers).
__device__ __forceinline__ void mx2_scales(const uint8_t *st, const Mx2Lds &o, uint32_t (&sa)[4], uint32_t (&sw)[2])
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint2 va = *reinterpret_cast<const uint2 *>(st + o.lsa + 256 * i);
        sa[i] = __builtin_amdgcn_perm(va.y, va.x, o.sel);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const uint2 vw = *reinterpret_cast<const uint2 *>(st + o.lsw + 256 * j);
        sw[j] = __builtin_amdgcn_perm(vw.y, vw.x, o.sel);
    }
}

__device__ __forceinline__ i32x8 mx2_wide(i32x4 v) { return __builtin_shufflevector(v, v, 0, 1, 2, 3, -1, -1, -1, -1); }

// acc[i][j] accumulates the transposed 32 x 32 block W_j A_i^T: lane l then holds
// output row 32 i + l % 32 and the 4 consecutive columns 32 j + 8 g + 4 (l / 32)
// + 0..3 in slots 4 g .. 4 g + 3, which the epilogue writes as one 8- or 16-byte
// piece.
template <int KS, int I0, int I1>
__device__ __forceinline__ void mx2_mfma(f32x16 (&acc)[4][2], const Mx2Frag &f, const uint32_t (&sa)[4],
                                         const uint32_t (&sw)[2])
{
#pragma unroll
    for (int i = I0; i < I1; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(mx2_wide(f.w[j]), mx2_wide(f.a[i]), acc[i][j],
                                                                        4, 4, KS, (int)sw[j], KS, (int)sa[i]);
}

// Interleave the 6 LDS reads of the next step with the 8 MFMAs of this one, one
// read after each of the first 6 MFMAs, so neither the reads' latency nor their
// registers pile up.
__device__ __forceinline__ void mx2_interleave()
{
#pragma unroll
    for (int t = 0; t < 6; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    }
    __builtin_amdgcn_sched_barrier(0);
}

// One stage: multiply the 256 K-elements in `cur` while the next stage lands in
// `oth`; then read step 0 of the next stage into f0 / sa / sw and start copying
// the stage after next into `cur` (`dn` holds the matrix descriptors, or empty
// ones when that stage does not exist).  Where no next stage exists the reads of
// `oth` fetch stale bytes that are never used.  The stage is one basic block
// whose instruction order the scheduling groups fix.
__device__ __forceinline__ void mx2_stage(uint8_t *cur, uint8_t *oth, int k_next2, const Mx2Dma &dn,
                                          const Mx2Lds &o, int wave, f32x16 (&acc)[4][2], Mx2Frag &f0,
                                          Mx2Frag &f1, uint32_t (&sa)[4], uint32_t (&sw)[2])
{
    mx2_frags(cur, o.la[1], o.lw[1], f1);
    mx2_mfma<0, 0, 4>(acc, f0, sa, sw);
    mx2_interleave();
    mx2_frags(cur, o.la[2], o.lw[2], f0);
    mx2_mfma<1, 0, 4>(acc, f1, sa, sw);
    mx2_interleave();
    mx2_frags(cur, o.la[3], o.lw[3], f1);
    mx2_mfma<2, 0, 4>(acc, f0, sa, sw);
    mx2_interleave();
    mx2_mfma<3, 0, 2>(acc, f1, sa, sw);
    __builtin_amdgcn_sched_barrier(0);
    // this wave's copy into `oth` has landed and its reads of `cur` returned; after
    // the barrier the same holds for every wave
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    uint32_t na[4], nw[2];
    mx2_scales(oth, o, na, nw);
    mx2_frags(oth, o.la[0], o.lw[0], f0);
    mx2_dma(cur, dn, k_next2, wave);
    mx2_mfma<3, 2, 4>(acc, f1, sa, sw);
#pragma unroll
    for (int i = 0; i < 4; ++i) sa[i] = na[i];
#pragma unroll
    for (int j = 0; j < 2; ++j) sw[j] = nw[j];
    __builtin_amdgcn_sched_barrier(0);
}

// Epilogue of the staged kernel.  The output tile passes through LDS so that
// every store instruction writes whole 512-byte (bf16) or 1 KiB (fp32) row
// runs.  Rows are padded by 16 bytes.  bf16: waves with wm = 0 stage tile rows
// 0..127 in s0 and waves with wm = 1 rows 128..255 in s1, in one round; fp32: the
// same split, 64 rows per wave row per round, two rounds.
template <typename T>
__device__ __forceinline__ void mx2_put(uint8_t *row, int col, const f32x16 &a, int g)
{
    if constexpr (sizeof(T) == 2) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        const bf16x4 v = {(__bf16)a[4 * g], (__bf16)a[4 * g + 1], (__bf16)a[4 * g + 2], (__bf16)a[4 * g + 3]};
        *reinterpret_cast<bf16x4 *>(row + 2 * col) = v;
    } else {
        *reinterpret_cast<f32x4 *>(row + 4 * col) = f32x4{a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
    }
}

// Store `rows` staged rows of width 256 elements (pitch bytes apart in `st`) to
// output rows m_first.. and columns n0..; the NT threads take 16-byte chunks in
// order.
template <typename T, int NT = 256, int COLS = 256>
__device__ __forceinline__ void mx2_flush(const uint8_t *st, int pitch, int rows, const MxGemmArgs &g, int m_first,
                                          int n0, int tid)
{
    constexpr int kPer = 16 / (int)sizeof(T);              // elements per chunk
    constexpr int kChunks = COLS / kPer;                   // chunks per row
    const int M = (int)g.M, N = (int)g.N;
    for (int q = tid; q < rows * kChunks; q += NT) {
        const int r = q / kChunks, ch = q % kChunks;
        const int m = m_first + r, n = n0 + ch * kPer;
        if (m >= M || n >= N) continue;
        const uint4 v = *reinterpret_cast<const uint4 *>(st + r * pitch + 16 * ch);
        T *dst = reinterpret_cast<T *>(g.c) + (int64_t)m * g.ldc + n;
        if (n + kPer <= N) {
            *reinterpret_cast<uint4 *>(dst) = v;
        } else {
            T e[kPer];
            __builtin_memcpy(e, &v, 16);
#pragma unroll
            for (int t = 0; t < kPer; ++t)
                if (n + t < N) dst[t] = e[t];
        }
    }
}

template <typename T>
__device__ __forceinline__ void mx2_epilogue(const f32x16 (&acc)[4][2], uint8_t *s0, uint8_t *s1, const MxGemmArgs &g,
                                             int m0, int n0, int wm, int wn, int lane, int tid)
{
    constexpr int pitch = 256 * (int)sizeof(T) + 16;
    constexpr int rounds = sizeof(T) == 2 ? 1 : 2;
    constexpr int rows = 128 / rounds;                     // staged rows per wave row per round
    static_assert(rows * pitch <= kSStage, "a staged half tile must fit one stage buffer");
    uint8_t *mine = wm ? s1 : s0;
#pragma unroll
    for (int rd = 0; rd < rounds; ++rd) {
#pragma unroll
        for (int i = rd * (4 / rounds); i < (rd + 1) * (4 / rounds); ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
#pragma unroll
                for (int gq = 0; gq < 4; ++gq)
                    mx2_put<T>(mine + (i * 32 - rd * rows + (lane & 31)) * pitch,
                               wn * 64 + j * 32 + 8 * gq + 4 * (lane >> 5), acc[i][j], gq);
                __builtin_amdgcn_sched_barrier(0);  // convert block by block: few live VGPRs
            }
        __syncthreads();
        mx2_flush<T, 512>(s0, pitch, rows, g, m0 + rd * rows, n0, tid);
        mx2_flush<T, 512>(s1, pitch, rows, g, m0 + 128 + rd * rows, n0, tid);
        if (rd + 1 < rounds) __syncthreads();
    }
}

template <typename OutT>
__global__ __launch_bounds__(512) void k_mx_gemm_2s(MxGemmArgs g)
{
    __shared__ __align__(16) uint8_t s0[kSStage];
    __shared__ __align__(16) uint8_t s1[kSStage];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int M = (int)g.M, N = (int)g.N, K = (int)g.K;
    const int tiles_m = (M + MBM - 1) / MBM, tiles_n = (N + MBN - 1) / MBN;
    int tm, tn;
    mx_tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * MBM, n0 = tn * MBN;
    const int nk = K / kSK;

    Mx2Dma d, dz;
    d.ra = mx2_rsrc(g.a_codes, g.M * (g.K / 2));
    d.rw = mx2_rsrc(g.w_codes, g.N * (g.K / 2));
    d.rsa = mx2_rsrc(g.a_scales, g.M * (g.K / 32));
    d.rsw = mx2_rsrc(g.w_scales, g.N * (g.K / 32));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = 256 * wave + 64 * i + lane;
        const int r = q >> 3;
        const int c = (q & 7) ^ ((r >> 1) & 7);
        d.a[i] = (uint32_t)min(m0 + r, M - 1) * (uint32_t)(K / 2) + 16 * c;
        d.w[i] = (uint32_t)min(n0 + r, N - 1) * (uint32_t)(K / 2) + 16 * c;
    }
    {
        const int q = 64 * wave + lane;
        d.as = (uint32_t)min(m0 + (q >> 1), M - 1) * (uint32_t)(K / 32) + 4 * (q & 1);
        d.ws = (uint32_t)min(n0 + (q >> 1), N - 1) * (uint32_t)(K / 32) + 4 * (q & 1);
    }
    Mx2Lds o;
    const int half = lane >> 5, x = ((lane & 31) >> 1) & 7;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        o.la[ks] = 128 * (wm * 128 + (lane & 31)) + 16 * ((2 * ks + half) ^ x);
        o.lw[ks] = kSTile + 128 * (wn * 64 + (lane & 31)) + 16 * ((2 * ks + half) ^ x);
    }
    o.lsa = 2 * kSTile + 8 * (wm * 128 + (lane & 31));
    o.lsw = 2 * kSTile + kSScl + 8 * (wn * 64 + (lane & 31));
    o.sel = half ? 0x07050301u : 0x06040200u;
    dz = d;
    dz.ra = mx2_rsrc(g.a_codes, 0);
    dz.rw = mx2_rsrc(g.w_codes, 0);
    dz.rsa = mx2_rsrc(g.a_scales, 0);
    dz.rsw = mx2_rsrc(g.w_scales, 0);

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

    // Stages t = 0 .. T-1 with T = nk rounded up to even: with nk odd, stage 0 is
    // an all-zero stage (its products add +0 to accumulators that start at +0)
    // and stage t holds K-elements [256 (t - 1), 256 t).
    const int ph = nk & 1, T = nk + ph;
    auto stage_k = [&](int t) { return max(t - ph, 0) * kSK; };
    auto stage_d = [&](int t) -> const Mx2Dma & { return (t >= ph && t < T) ? d : dz; };
    mx2_dma(s0, stage_d(0), stage_k(0), wave);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    mx2_dma(s1, stage_d(1), stage_k(1), wave);
    Mx2Frag f0, f1;
    uint32_t sa[4], sw[2];
    mx2_scales(s0, o, sa, sw);
    mx2_frags(s0, o.la[0], o.lw[0], f0);
    for (int t = 0; t < T; t += 2) {
        mx2_stage(s0, s1, stage_k(t + 2), stage_d(t + 2), o, wave, acc, f0, f1, sa, sw);
        mx2_stage(s1, s0, stage_k(t + 3), stage_d(t + 3), o, wave, acc, f0, f1, sa, sw);
    }

    __builtin_amdgcn_s_waitcnt(0);  // the empty copies issued by the last stages have landed
    __syncthreads();  // both stages free: stage the output in them
    // the lane index is recomputed rather than kept live through the main loop
    const int lane_e = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    mx2_epilogue<OutT>(acc, s0, s1, g, m0, n0, wm, wn, lane_e, 64 * wave + lane_e);
}

// ---- generic path (K % 128 != 0): double-buffered register prefetch ----

struct MxPrefetch {
    uint4 a[4], w[4];
    uint32_t sa, sw;
};

template <bool ALIGNED>
__device__ __forceinline__ uint32_t ld_scale4(const uint8_t *sp, int k0, int K)
{
    if (ALIGNED) return *reinterpret_cast<const uint32_t *>(sp);
    uint32_t s = 0;
    for (int b = 0; b < 4; ++b)
        if (k0 + 32 * b < K) s |= (uint32_t)sp[b] << (8 * b);
    return s;
}

template <bool ALIGNED>
__device__ __forceinline__ void mx_load(MxPrefetch &p, const MxGemmArgs &g, int64_t m0, int64_t n0,
                                        int k0, int tid)
{
    const int K = (int)g.K;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int id = i * 256 + tid;
        const int row = id >> 2, ch = id & 3;
        const int k = k0 + ch * 32;
        const int64_t m = m0 + row, n = n0 + row;
        p.a[i] = uint4{0u, 0u, 0u, 0u};
        p.w[i] = uint4{0u, 0u, 0u, 0u};
        if (k < K) {
            if (m < g.M) p.a[i] = *reinterpret_cast<const uint4 *>(g.a_codes + m * (K / 2) + k / 2);
            if (n < g.N) p.w[i] = *reinterpret_cast<const uint4 *>(g.w_codes + n * (K / 2) + k / 2);
        }
    }
    p.sa = 0;
    p.sw = 0;
    const int64_t m = m0 + tid, n = n0 + tid;
    if (m < g.M) p.sa = ld_scale4<ALIGNED>(g.a_scales + m * (K / 32) + k0 / 32, k0, K);
    if (n < g.N) p.sw = ld_scale4<ALIGNED>(g.w_scales + n * (K / 32) + k0 / 32, k0, K);
}

__device__ __forceinline__ void mx_store(uint8_t *As, uint8_t *Ws, uint32_t *Sa, uint32_t *Sw,
                                         const MxPrefetch &p, int tid)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int id = i * 256 + tid;
        const int row = id >> 2, ch = id & 3;
        *reinterpret_cast<uint4 *>(As + mswz(row, ch)) = p.a[i];
        *reinterpret_cast<uint4 *>(Ws + mswz(row, ch)) = p.w[i];
    }
    Sa[tid] = p.sa;
    Sw[tid] = p.sw;
}

template <bool ALIGNED>
__global__ __launch_bounds__(256) void k_mx_gemm(MxGemmArgs g)
{
    extern __shared__ __align__(16) uint8_t msmem[];
    constexpr int kTileBytes = MBM * kRowBytes;  // 16 KiB
    // buffer b: A codes at b * kTileBytes, W codes at (2 + b) * kTileBytes, then the
    // scale dwords: A buffer b at b * MBM, W buffer b at 2 * MBM + b * MBN
    uint8_t *const Abase = msmem;
    uint8_t *const Wbase = msmem + 2 * kTileBytes;
    uint32_t *const Sbase = reinterpret_cast<uint32_t *>(msmem + 4 * kTileBytes);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int M = (int)g.M, N = (int)g.N, K = (int)g.K;
    const int tiles_m = (M + MBM - 1) / MBM, tiles_n = (N + MBN - 1) / MBN;
    int tm, tn;
    mx_tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * MBM, n0 = (int64_t)tn * MBN;

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

    MxPrefetch p;
    const int nk = (K + MBK - 1) / MBK;
    mx_load<ALIGNED>(p, g, m0, n0, 0, tid);
    mx_store(Abase, Wbase, Sbase, Sbase + 2 * MBM, p, tid);
    __syncthreads();

    const int half = lane >> 5;
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        const uint8_t *Ac = Abase + cur * kTileBytes, *Wc = Wbase + cur * kTileBytes;
        const uint32_t *Sac = Sbase + cur * MBM, *Swc = Sbase + 2 * MBM + cur * MBN;
        if (more) mx_load<ALIGNED>(p, g, m0, n0, (kt + 1) * MBK, tid);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int ch = ks * 2 + half;           // this lane's 32 K-elements = MX block ch
            i32x8 af[4], wf[4];
            int sa[4], sw[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = wm * 128 + i * 32 + (lane & 31);
                const uint4 v = *reinterpret_cast<const uint4 *>(Ac + mswz(row, ch));
                af[i] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
                sa[i] = (int)((Sac[row] >> (8 * ch)) & 0xFFu);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = wn * 128 + j * 32 + (lane & 31);
                const uint4 v = *reinterpret_cast<const uint4 *>(Wc + mswz(row, ch));
                wf[j] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
                sw[j] = (int)((Swc[row] >> (8 * ch)) & 0xFFu);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        af[i], wf[j], acc[i][j], 4, 4, 0, sa[i], 0, sw[j]);
        }
        if (more)
            mx_store(Abase + (cur ^ 1) * kTileBytes, Wbase + (cur ^ 1) * kTileBytes,
                     Sbase + (cur ^ 1) * MBM, Sbase + 2 * MBM + (cur ^ 1) * MBN, p, tid);
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int64_t m = m0 + wm * 128 + i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
            if (m >= M) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t n = n0 + wn * 128 + j * 32 + (lane & 31);
                if (n >= N) continue;
                const float o = acc[i][j][e];
                if (g.c_bf16)
                    reinterpret_cast<uint16_t *>(g.c)[m * g.ldc + n] = (uint16_t)f32_to_bf16_rne(o);
                else
                    reinterpret_cast<float *>(g.c)[m * g.ldc + n] = o;
            }
        }
    }
}

constexpr size_t kMxLds = (size_t)4 * MBM * kRowBytes + (size_t)2 * (MBM + MBN) * 4;  // 68 KiB

template <bool ALIGNED>
static fp4_status launch_mx(const MxGemmArgs &g, hipStream_t st)
{
    static std::atomic<uint64_t> lds_set{0};  // per device
    if (!set_max_lds_once((const void *)k_mx_gemm<ALIGNED>, (int)kMxLds, lds_set)) return FP4_ERR_HIP;
    const int tiles = (int)(((g.M + MBM - 1) / MBM) * ((g.N + MBN - 1) / MBN));
    hipLaunchKernelGGL(k_mx_gemm<ALIGNED>, dim3(tiles), dim3(256), kMxLds, st, g);
    return hipGetLastError() == hipSuccess ? FP4_OK : FP4_ERR_HIP;
}

// ---- W4A8: MXFP8 activations x MXFP4 weights (K % 128 == 0) -------------
//
// W4A8 (edge-FP4 article, eefocus.com: an NPU with native W4A8, weights in FP4
// and activations in FP8), with both operands in OCP MX form: A E4M3FN bytes
// and W E2M1 nibbles, each with an E8M0 byte per 32 K-elements.  gfx950's
// v_mfma_scale_f32_32x32x64_f8f6f4 takes the two formats side by side (source 0
// FP4, source 1 FP8).  Of the instruction's 64 K-values, lane half h (lanes
// 32 h ..) supplies, for its row, the FP4 values 32 h .. 32 h + 31 as 16 bytes,
// but the FP8 values 16 h .. 16 h + 15 and 32 + 16 h .. 32 + 16 h + 15 as its two
// 16-byte halves; the E8M0 byte a lane half gives applies to K-block h of
// either operand.  Products are exact, the accumulation fp32.
//
// 256 x 256 tiles, 8 waves (two per SIMD) as 4 (M) x 2 (N) blocks of 64 x 128
// (the 32-byte FP8 fragments make the A side the expensive one to hold and read),
// acc[i][j] = W_j A_i^T as in the MXFP4 kernel.  Three LDS stages of 128 K-elements, each its own LDS object,
// fed by buffer-to-LDS DMA: A [256][128 B] (16-byte chunk c of row r at slot
// 8 r + (c ^ ((r >> 1) & 7))), W [256][64 B] (chunk c at 4 r + (c ^ ((r >> 2) & 3))),
// and each operand's 4 E8M0 bytes per row.  Those swizzles make the 16 lanes of
// each fragment read hit 16 different 16-byte bank groups.  A stage is two MFMA
// steps of 64 K; step 1's fragments are read under step 0's MFMAs, and after the
// barrier that frees the stage (inside step 1) the next stage's step 0 is read
// and the copy of the stage three ahead starts.
constexpr int kA8K = 128;                  // K elements per stage
constexpr int kA8A = 0;                    // A fp8 [256][128]
constexpr int kA8W = 256 * 128;            // W fp4 [256][64]
constexpr int kA8SA = kA8W + 256 * 64;     // A scales [256][4]
constexpr int kA8SW = kA8SA + 1024;        // W scales [256][4]
constexpr int kA8Stage = kA8SW + 1024;     // 51,200 bytes
constexpr int kA8Dma = 4 + 2 + 1;          // copies per wave per stage
constexpr uint32_t kA8Out = 0x80000000u;   // an offset past every descriptor's size
constexpr int kA8EpiPitch16 = 256 * 2 + 16, kA8EpiPitch32 = 256 * 4 + 16;
static_assert(64 * kA8EpiPitch16 <= kA8Stage && 32 * kA8EpiPitch32 <= kA8Stage, "epilogue staging");

// Per-lane source offsets of a wave's copies: A code slot q = 256 wave + 64 i +
// lane (row q / 8), W code slot q = 128 wave + 64 i + lane (row q / 4), and one
// scale dword: waves 0..3 copy A's rows 64 wave + lane, waves 4..7 W's rows
// 64 (wave - 4) + lane, into bytes kA8SA + 256 wave + 4 lane of the stage.  Stage
// t's bytes start t * w_step past a W offset and t * s_step past this wave's
// scale offset: 64 and 4 for row-major W, N * 64 and N * 4 for segment-major W
// (whose 128-element segments are contiguous panels; A stays row-major).
struct A8Dma {
    __amdgpu_buffer_rsrc_t ra, rw, rs;
    uint32_t a[4], w[2], s;
    uint32_t w_step, s_step;
};

__device__ __forceinline__ void a8_dma(uint8_t *st, const A8Dma &d, int k0, int wave)
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(d.ra, (mx_lds_void *)(st + kA8A + 16 * (256 * wave + 64 * i)), 16,
                                                 (int)d.a[i], k0, 0, 0);
    const int t = k0 / kA8K;
#pragma unroll
    for (int i = 0; i < 2; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rw, (mx_lds_void *)(st + kA8W + 16 * (128 * wave + 64 * i)), 16,
                                                 (int)d.w[i], t * (int)d.w_step, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rs, (mx_lds_void *)(st + kA8SA + 256 * wave), 4, (int)d.s,
                                             t * (int)d.s_step, 0, 0);
}

// per-lane LDS offsets: A row wm 64 + l, W row wn 128 + l (l = lane % 32, half
// h = lane / 32); fragment i / j adds 32 rows (4096 / 2048 bytes)
struct A8Lds {
    uint32_t a[2][2];  // [step][16-byte half p] A chunk 4 ks + 2 p + h
    uint32_t w[2];     // [step] W chunk 2 ks + h
    uint32_t sa, sw;   // the row's 4 scale bytes
    uint32_t hsh;      // 8 h: this lane's scale bytes are bits hsh.. and 16 + hsh..
};

struct A8Frag {
    i32x8 a[2];
    i32x4 w[4];
};

template <int KS>
__device__ __forceinline__ void a8_frags(const uint8_t *st, const A8Lds &o, A8Frag &f)
{
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const i32x4 lo = *reinterpret_cast<const i32x4 *>(st + o.a[KS][0] + 4096 * i);
        const i32x4 hi = *reinterpret_cast<const i32x4 *>(st + o.a[KS][1] + 4096 * i);
        f.a[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) f.w[j] = *reinterpret_cast<const i32x4 *>(st + o.w[KS] + 2048 * j);
}

// the lane's E8M0 bytes of the stage: byte 0 = step 0's block, byte 2 = step 1's
__device__ __forceinline__ void a8_scales(const uint8_t *st, const A8Lds &o, uint32_t (&sa)[2], uint32_t (&sw)[4])
{
#pragma unroll
    for (int i = 0; i < 2; ++i)
        sa[i] = (*reinterpret_cast<const uint32_t *>(st + o.sa + 128 * i) >> o.hsh) & 0x00FF00FFu;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        sw[j] = (*reinterpret_cast<const uint32_t *>(st + o.sw + 128 * j) >> o.hsh) & 0x00FF00FFu;
}

template <int KS>
__device__ __forceinline__ void a8_mfma(f32x16 (&acc)[2][4], const A8Frag &f, const uint32_t (&sa)[2],
                                        const uint32_t (&sw)[4])
{
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(mx2_wide(f.w[j]), f.a[i], acc[i][j], 4, 0,
                                                                        2 * KS, (int)sw[j], 2 * KS, (int)sa[i]);
}

// the 8 fragment reads of step 1 under the 8 MFMAs of step 0, one after each
__device__ __forceinline__ void a8_interleave()
{
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    }
    __builtin_amdgcn_sched_barrier(0);
}

// One stage t (in `cur`, stage t + 1 in `nxt`); f0 / sa / sw hold step 0 of t.
__device__ __forceinline__ void a8_stage(uint8_t *cur, const uint8_t *nxt, int t, int nk, const A8Dma &d,
                                         const A8Dma &dz, const A8Lds &o, int wave, f32x16 (&acc)[2][4], A8Frag &f0,
                                         A8Frag &f1, uint32_t (&sa)[2], uint32_t (&sw)[4])
{
    a8_frags<1>(cur, o, f1);
    a8_mfma<0>(acc, f0, sa, sw);
    a8_interleave();
    __builtin_amdgcn_s_waitcnt((kA8Dma & 15) | ((kA8Dma >> 4) << 14) | (7 << 4) | (15 << 8));  // stage t + 1 landed
    __builtin_amdgcn_s_waitcnt((0xF) | (0x3 << 14) | (7 << 4));                                // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
    uint32_t na[2], nw[4];
    a8_scales(nxt, o, na, nw);
    a8_frags<0>(nxt, o, f0);
    a8_dma(cur, t + 3 < nk ? d : dz, (t + 3 < nk ? t + 3 : 0) * kA8K, wave);
    a8_mfma<1>(acc, f1, sa, sw);
    // the next stage's 14 reads and this stage's 7 copies spread over step 1's 8
    // MFMAs (two reads, an MFMA, a copy): a burst of copies would hold back the
    // MFMAs behind it in the wave's instruction stream (545 us instead of 583 us
    // at M = 8192)
#pragma unroll
    for (int q = 0; q < kA8Dma; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM: a copy
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8 - kA8Dma, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 2; ++i) sa[i] = na[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) sw[j] = nw[j];
}

// Epilogue: tile rows 0..127 (waves wm = 0, 1) pass through s0, rows 128..255
// (wm = 2, 3) through s1, in rounds of R rows (rows padded by 16 bytes), each
// round then stored as whole-row 16-byte pieces.
template <typename T>
__device__ __forceinline__ void a8_epilogue(const f32x16 (&acc)[2][4], uint8_t *s0, uint8_t *s1,
                                            const MxGemmArgs &g, int m0, int n0, int wm, int wn, int lane, int tid)
{
    constexpr int es = (int)sizeof(T);
    constexpr int pitch = es == 2 ? kA8EpiPitch16 : kA8EpiPitch32;
    constexpr int R = es == 2 ? 64 : 32;
    uint8_t *mine = wm >= 2 ? s1 : s0;
    const int half_row0 = 64 * (wm & 1);  // the wave's first row within its 128-row half
#pragma unroll
    for (int rd = 0; rd < 128 / R; ++rd) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = half_row0 + 32 * i - rd * R;  // wave-uniform
            if (r >= 0 && r < R) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq)
                        mx2_put<T>(mine + (r + (lane & 31)) * pitch, wn * 128 + j * 32 + 8 * gq + 4 * (lane >> 5),
                                   acc[i][j], gq);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        __syncthreads();
        mx2_flush<T, 512>(s0, pitch, R, g, m0 + rd * R, n0, tid);
        mx2_flush<T, 512>(s1, pitch, R, g, m0 + 128 + rd * R, n0, tid);
        __syncthreads();
    }
}

template <typename OutT>
__global__ __launch_bounds__(512) void k_mx_gemm_w4a8(MxGemmArgs g)
{
    __shared__ __align__(16) uint8_t s0[kA8Stage];
    __shared__ __align__(16) uint8_t s1[kA8Stage];
    __shared__ __align__(16) uint8_t s2[kA8Stage];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int M = (int)g.M, N = (int)g.N, K = (int)g.K;
    const int tiles_m = (M + MBM - 1) / MBM, tiles_n = (N + MBN - 1) / MBN;
    int tm, tn;
    mx_tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * MBM, n0 = tn * MBN;
    const int nk = K / kA8K;

    A8Dma d, dz;
    d.ra = mx2_rsrc(g.a_codes, g.M * g.K);
    d.rw = mx2_rsrc(g.w_codes, g.N * (g.K / 2));
    d.rs = wave < 4 ? mx2_rsrc(g.a_scales, g.M * (g.K / 32)) : mx2_rsrc(g.w_scales, g.N * (g.K / 32));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = 256 * wave + 64 * i + lane;
        const int r = q >> 3, c = (q & 7) ^ ((r >> 1) & 7);
        d.a[i] = m0 + r < M ? (uint32_t)(m0 + r) * (uint32_t)K + 16 * c : kA8Out;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int q = 128 * wave + 64 * i + lane;
        const int r = q >> 2, c = (q & 3) ^ ((r >> 2) & 3);
        d.w[i] = n0 + r < N ? (uint32_t)(n0 + r) * (uint32_t)(g.w_seg ? 64 : K / 2) + 16 * c : kA8Out;
    }
    {
        const int r = 64 * (wave & 3) + lane;
        if (wave < 4) d.s = m0 + r < M ? (uint32_t)(m0 + r) * (uint32_t)(K / 32) : kA8Out;
        else d.s = n0 + r < N ? (uint32_t)(n0 + r) * (uint32_t)(g.w_seg ? 4 : K / 32) : kA8Out;
    }
    d.w_step = g.w_seg ? (uint32_t)N * 64u : 64u;
    d.s_step = g.w_seg && wave >= 4 ? (uint32_t)N * 4u : 4u;
    dz = d;
    dz.ra = mx2_rsrc(g.a_codes, 0);
    dz.rw = mx2_rsrc(g.w_codes, 0);
    dz.rs = mx2_rsrc(g.a_scales, 0);

    A8Lds o;
    {
        const int h = lane >> 5, l = lane & 31;
        const int ra = wm * 64 + l, rw = wn * 128 + l;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int p = 0; p < 2; ++p) o.a[ks][p] = kA8A + 128 * ra + 16 * ((4 * ks + 2 * p + h) ^ ((ra >> 1) & 7));
            o.w[ks] = kA8W + 64 * rw + 16 * ((2 * ks + h) ^ ((rw >> 2) & 3));
        }
        o.sa = kA8SA + 4 * ra;
        o.sw = kA8SW + 4 * rw;
        o.hsh = 8 * h;
    }

    f32x16 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

    a8_dma(s0, d, 0, wave);
    a8_dma(s1, nk > 1 ? d : dz, nk > 1 ? kA8K : 0, wave);
    a8_dma(s2, nk > 2 ? d : dz, nk > 2 ? 2 * kA8K : 0, wave);
    __builtin_amdgcn_s_waitcnt(((2 * kA8Dma) & 15) | (((2 * kA8Dma) >> 4) << 14) | (7 << 4) | (15 << 8));
    asm volatile("s_barrier" ::: "memory");
    A8Frag f0, f1;
    uint32_t sa[2], sw[4];
    a8_scales(s0, o, sa, sw);
    a8_frags<0>(s0, o, f0);
    const int nfull = nk - nk % 3;
    for (int t = 0; t < nfull; t += 3) {
        a8_stage(s0, s1, t, nk, d, dz, o, wave, acc, f0, f1, sa, sw);
        a8_stage(s1, s2, t + 1, nk, d, dz, o, wave, acc, f0, f1, sa, sw);
        a8_stage(s2, s0, t + 2, nk, d, dz, o, wave, acc, f0, f1, sa, sw);
    }
    if (nk % 3 >= 1) a8_stage(s0, s1, nfull, nk, d, dz, o, wave, acc, f0, f1, sa, sw);
    if (nk % 3 == 2) a8_stage(s1, s2, nfull + 1, nk, d, dz, o, wave, acc, f0, f1, sa, sw);

    __builtin_amdgcn_s_waitcnt(0);  // the last (empty) copies landed
    __syncthreads();
    const int lane_e = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    a8_epilogue<OutT>(acc, s0, s1, g, m0, n0, wm, wn, lane_e, 64 * wave + lane_e);
}

fp4_status launch_mxfp4_gemm_w4a8(const MxGemmArgs &g, hipStream_t st)
{
    // 32-bit byte offsets into A (M K bytes) and W
    if (g.K % kA8K != 0 || g.M * g.K >= (int64_t(1) << 31) || g.N * (g.K / 2) >= (int64_t(1) << 31))
        return FP4_ERR_SHAPE;
    const int tiles = (int)(((g.M + MBM - 1) / MBM) * ((g.N + MBN - 1) / MBN));
    if (g.c_bf16)
        hipLaunchKernelGGL((k_mx_gemm_w4a8<__bf16>), dim3(tiles), dim3(512), 0, st, g);
    else
        hipLaunchKernelGGL((k_mx_gemm_w4a8<float>), dim3(tiles), dim3(512), 0, st, g);
    return hipGetLastError() == hipSuccess ? FP4_OK : FP4_ERR_HIP;
}

// ---- segment-major operands: a ring of four LDS slots of 128 K-elements ----
//
// Both operands in the segment-major layout (the MXFP4 decode layout): for each
// 128-element K segment s, every row's 64 code bytes at (s rows + r) 64 and its
// 4 E8M0 bytes at (s rows + r) 4.  One segment of a 256-row panel is then 16 KiB
// of contiguous bytes, so a slot of 128 K costs whole cache lines; in the
// row-major layout the same slot is 64-byte halves of lines, which the memory
// system moves at three quarters of the rate (a copy-only kernel with the GEMM's
// pattern: 239 us against 178 us).  With 34 KiB slots four fit in LDS: while
// slot s is multiplied, slots s + 1 and s + 2 are landing and slot s + 3 is being
// copied, its 5 copies per wave spread among slot s's MFMAs; a copy issued in a
// burst holds back the MFMAs behind it in the wave's instruction stream.
//
// 8 waves as in k_mx_gemm_2s (2 x 4 blocks of 128 x 64).  Slot layout: codes
// [256][64] per operand (16-byte chunk c of row r at slot c ^ ((r >> 2) & 3)),
// then each operand's [256][4] scale bytes.  Rows past the matrix read the last
// row (their products land only in outputs that are never stored); slots past
// the end are filled through size-0 descriptors (zeros).  Slot count T is nk
// rounded up to a multiple of 4, the first T - nk slots being such zero slots.
constexpr int kQK = 128;                         // K elements per slot
constexpr int kQTile = 256 * 64;                 // 16 KiB of codes per operand
constexpr int kQScl = 256 * 4;                   // 1 KiB of scale bytes per operand
constexpr int kQSlot = 2 * kQTile + 2 * kQScl;   // 34,816 bytes
constexpr int kQDma = 5;                         // copies per wave per slot

// per-lane source offsets within a segment: A / W code slot q = 128 wave + 64 i +
// lane (row q / 4); one scale dword, waves 0..3 for A rows 64 wave + lane, waves
// 4..7 for W rows 64 (wave - 4) + lane.  A segment's bytes start at s * seg_a /
// seg_w / seg_s (the scalar offset of each copy).
struct MqDma {
    __amdgpu_buffer_rsrc_t ra, rw, rs;
    uint32_t a[2], w[2], s;
    uint32_t seg_a, seg_w, seg_s;
};

template <int P>
__device__ __forceinline__ void mq_dma(uint8_t *st, const MqDma &d, int seg, int wave)
{
    if constexpr (P < 2)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(d.ra, (mx_lds_void *)(st + 16 * (128 * wave + 64 * P)), 16,
                                                 (int)d.a[P], seg * (int)d.seg_a, 0, 0);
    else if constexpr (P < 4)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rw, (mx_lds_void *)(st + kQTile + 16 * (128 * wave + 64 * (P - 2))),
                                                 16, (int)d.w[P - 2], seg * (int)d.seg_w, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rs, (mx_lds_void *)(st + 2 * kQTile + 256 * wave), 4, (int)d.s,
                                                 seg * (int)d.seg_s, 0, 0);
}

__device__ __forceinline__ void mq_dma_all(uint8_t *st, const MqDma &d, int seg, int wave)
{
    mq_dma<0>(st, d, seg, wave);
    mq_dma<1>(st, d, seg, wave);
    mq_dma<2>(st, d, seg, wave);
    mq_dma<3>(st, d, seg, wave);
    mq_dma<4>(st, d, seg, wave);
}

// LDS offsets one lane reads within a slot: A fragment (i, ks) at la[ks] + 2048 i,
// W fragment (j, ks) at lw[ks] + 2048 j; scale dwords at lsa + 128 i, lsw + 128 j
struct MqLds {
    uint32_t la[2], lw[2], lsa, lsw, hsh;
};

template <int NJ>
__device__ __forceinline__ void mq_frags(const uint8_t *st, uint32_t la, uint32_t lw, Mx2Frag &f)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) f.a[i] = *reinterpret_cast<const i32x4 *>(st + la + 2048 * i);
#pragma unroll
    for (int j = 0; j < NJ; ++j) f.w[j] = *reinterpret_cast<const i32x4 *>(st + lw + 2048 * j);
}

// the lane's E8M0 bytes of the slot: byte 0 = step 0's block (2 * 0 + h), byte 2 =
// step 1's (2 + h), h the lane half
template <int NJ>
__device__ __forceinline__ void mq_scales(const uint8_t *st, const MqLds &o, uint32_t (&sa)[4], uint32_t (&sw)[2])
{
#pragma unroll
    for (int i = 0; i < 4; ++i) sa[i] = (*reinterpret_cast<const uint32_t *>(st + o.lsa + 128 * i) >> o.hsh) & 0x00FF00FFu;
#pragma unroll
    for (int j = 0; j < NJ; ++j) sw[j] = (*reinterpret_cast<const uint32_t *>(st + o.lsw + 128 * j) >> o.hsh) & 0x00FF00FFu;
}

template <int KS, int I0, int I1, int NJ>
__device__ __forceinline__ void mq_mfma(f32x16 (&acc)[4][NJ], const Mx2Frag &f, const uint32_t (&sa)[4],
                                        const uint32_t (&sw)[2])
{
#pragma unroll
    for (int i = I0; i < I1; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(mx2_wide(f.w[j]), mx2_wide(f.a[i]), acc[i][j],
                                                                        4, 4, 2 * KS, (int)sw[j], 2 * KS, (int)sa[i]);
}

// Slot s: multiply `cur` (f0 / sa / sw hold its step 0); copy segment `seg` (slot
// s + 3) into `dst`, which the previous barrier freed, spread among the MFMAs; at
// the barrier slot s + 1 (`nxt`) must have landed, while the 10 copies of slots
// s + 2 and s + 3 may still be in flight.  One basic block.
template <int NJ>
__device__ __forceinline__ void mq_slot(const uint8_t *cur, const uint8_t *nxt, uint8_t *dst, const MqDma &d,
                                        int seg, const MqLds &o, int wave, f32x16 (&acc)[4][NJ], Mx2Frag &f0,
                                        Mx2Frag &f1, uint32_t (&sa)[4], uint32_t (&sw)[2])
{
    constexpr int nm = 4 * NJ;  // MFMAs per step
    // step 0: nm MFMAs, the 4 + NJ reads of step 1's fragments, 3 copies
    mq_frags<NJ>(cur, o.la[1], o.lw[1], f1);
    mq_mfma<0, 0, 4, NJ>(acc, f0, sa, sw);
    mq_dma<0>(dst, d, seg, wave);
    mq_dma<1>(dst, d, seg, wave);
    mq_dma<2>(dst, d, seg, wave);
#pragma unroll
    for (int t = 0; t < nm; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                       // MFMA
        if (t < 4 + NJ) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);       // DS read
        if (t == 1 || t == nm / 2 || t == nm - 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // copy
    }
    __builtin_amdgcn_sched_barrier(0);
    // step 1, first half: nm / 2 MFMAs, 2 copies
    mq_mfma<1, 0, 2, NJ>(acc, f1, sa, sw);
    mq_dma<3>(dst, d, seg, wave);
    mq_dma<4>(dst, d, seg, wave);
#pragma unroll
    for (int t = 0; t < nm / 2; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (t == 0 || t == nm / 4) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // slot s + 1 has landed (vmcnt 10) and this wave's reads of `cur` returned; the
    // barrier extends both to every wave
    __builtin_amdgcn_s_waitcnt(((2 * kQDma) & 15) | (7 << 4));
    asm volatile("s_barrier" ::: "memory");
    uint32_t na[4], nw[2];
    mq_scales<NJ>(nxt, o, na, nw);
    mq_frags<NJ>(nxt, o.la[0], o.lw[0], f0);
    mq_mfma<1, 2, 4, NJ>(acc, f1, sa, sw);
#pragma unroll
    for (int i = 0; i < 4; ++i) sa[i] = na[i];
#pragma unroll
    for (int j = 0; j < NJ; ++j) sw[j] = nw[j];
    __builtin_amdgcn_sched_barrier(0);
}

// Epilogue through the four slots: bf16 stages 64 tile rows per slot (slots 0, 1
// rows 0..127 from the waves with wm = 0, slots 2, 3 rows 128..255), one round;
// fp32 32 rows per slot, two rounds.
template <typename T, int NJ>
__device__ __forceinline__ void mq_epilogue(const f32x16 (&acc)[4][NJ], uint8_t *q0, uint8_t *q1, uint8_t *q2,
                                            uint8_t *q3, const MxGemmArgs &g, int m0, int n0, int wm, int wn,
                                            int lane, int tid)
{
    constexpr int pitch = 256 * (int)sizeof(T) + 16;
    constexpr int rows = sizeof(T) == 2 ? 64 : 32;  // rows per slot per round
    constexpr int rounds = sizeof(T) == 2 ? 1 : 2;
    static_assert(rows * pitch <= kQSlot, "a slot holds a round's rows");
#pragma unroll
    for (int rd = 0; rd < rounds; ++rd) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (sizeof(T) == 4 && i / 2 != rd) continue;
            const int rr = sizeof(T) == 2 ? 32 * i : 32 * i - 64 * rd;  // row within the round's two slots
            const int sub = rr / rows;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                uint8_t *slot = wm ? (sub ? q3 : q2) : (sub ? q1 : q0);
#pragma unroll
                for (int gq = 0; gq < 4; ++gq)
                    mx2_put<T>(slot + (rr % rows + (lane & 31)) * pitch,
                               wn * 32 * NJ + j * 32 + 8 * gq + 4 * (lane >> 5), acc[i][j], gq);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        __syncthreads();
        const int mr = m0 + (sizeof(T) == 4 ? 64 * rd : 0);
        mx2_flush<T, 512, 128 * NJ>(q0, pitch, rows, g, mr, n0, tid);
        mx2_flush<T, 512, 128 * NJ>(q1, pitch, rows, g, mr + rows, n0, tid);
        mx2_flush<T, 512, 128 * NJ>(q2, pitch, rows, g, mr + 128, n0, tid);
        mx2_flush<T, 512, 128 * NJ>(q3, pitch, rows, g, mr + 128 + rows, n0, tid);
        if (rd + 1 < rounds) __syncthreads();
    }
}

// AROW / WROW: that operand is row-major instead (codes [rows][K/2], E8M0
// [rows][K/32]): a row's 128-K segment is then the 64 bytes at row K/2 + 64 s and
// its 4 scale bytes at row K/32 + 4 s, so only the copies' row stride and
// segment step change; the slots, fragments and contraction order are the same,
// and so is every output bit.
// TN = 128: tiles of 256 x 128 for a last round that 256 x 256 tiles would leave
// half empty; each wave then owns 128 x 32, the copies of W rows 128..255 and
// their scale bytes read nothing (they keep every wave's copy count, which the
// slot waits count), and the same K steps are contracted in the same order.
constexpr uint32_t kMqOut = 0x80000000u;  // an offset past every descriptor's size
template <typename OutT, bool AROW = false, bool WROW = false, int TN = 256>
__global__ __launch_bounds__(512) void k_mx_gemm_seg(MxGemmArgs g)
{
    static_assert(TN == 256 || TN == 128, "tile width");
    constexpr int NJ = TN / 128;  // 32-column blocks per wave
    __shared__ __align__(16) uint8_t q0[kQSlot];
    __shared__ __align__(16) uint8_t q1[kQSlot];
    __shared__ __align__(16) uint8_t q2[kQSlot];
    __shared__ __align__(16) uint8_t q3[kQSlot];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int M = (int)g.M, N = (int)g.N, K = (int)g.K;
    const int tiles_m = (M + MBM - 1) / MBM, tiles_n = (N + TN - 1) / TN;
    int tm, tn;
    mx_tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * MBM, n0 = tn * TN;
    const int nk = K / kQK;
    // W rows w_row0 .. w_row0 + N - 1 of a weight of wrows rows
    const int w_row0 = (int)g.w_row0, wrows = (int)(g.w_rows ? g.w_rows : g.N);

    MqDma d, dz;
    d.ra = mx2_rsrc(g.a_codes, g.M * (g.K / 2));
    d.rw = mx2_rsrc(g.w_codes, (int64_t)wrows * (g.K / 2));
    d.rs = wave < 4 ? mx2_rsrc(g.a_scales, g.M * (g.K / 32)) : mx2_rsrc(g.w_scales, (int64_t)wrows * (g.K / 32));
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int q = 128 * wave + 64 * i + lane;
        const int r = q >> 2;
        const int c = (q & 3) ^ ((r >> 2) & 3);
        d.a[i] = (uint32_t)min(m0 + r, M - 1) * (AROW ? (uint32_t)(K / 2) : 64u) + 16 * c;
        d.w[i] = r < TN ? (uint32_t)(w_row0 + min(n0 + r, N - 1)) * (WROW ? (uint32_t)(K / 2) : 64u) + 16 * c
                        : kMqOut;
    }
    const bool srow = wave < 4 ? AROW : WROW;  // this wave copies A's (waves 0-3) or W's scale bytes
    {
        const int r = 64 * (wave & 3) + lane;
        const uint32_t step = srow ? (uint32_t)(K / 32) : 4u;
        d.s = wave < 4 ? (uint32_t)min(m0 + r, M - 1) * step
                       : (r < TN ? (uint32_t)(w_row0 + min(n0 + r, N - 1)) * step : kMqOut);
    }
    d.seg_a = AROW ? 64u : (uint32_t)M * 64u;
    d.seg_w = WROW ? 64u : (uint32_t)wrows * 64u;
    d.seg_s = srow ? 4u : (uint32_t)(wave < 4 ? M : wrows) * 4u;
    dz = d;
    dz.ra = mx2_rsrc(g.a_codes, 0);
    dz.rw = mx2_rsrc(g.w_codes, 0);
    dz.rs = mx2_rsrc(g.a_scales, 0);

    MqLds o;
    {
        const int h = lane >> 5, l = lane & 31;
        const int ra = wm * 128 + l, rw = wn * 32 * NJ + l;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            o.la[ks] = 64 * ra + 16 * ((2 * ks + h) ^ ((ra >> 2) & 3));
            o.lw[ks] = kQTile + 64 * rw + 16 * ((2 * ks + h) ^ ((rw >> 2) & 3));
        }
        o.lsa = 2 * kQTile + 4 * ra;
        o.lsw = 2 * kQTile + kQScl + 4 * rw;
        o.hsh = 8 * h;
    }

    f32x16 acc[4][NJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{};

    const int T = (nk + 3) & ~3, ph = T - nk;
    auto seg_of = [&](int t) { return max(t - ph, 0); };
    auto slot_d = [&](int t) -> const MqDma & { return (t >= ph && t < T) ? d : dz; };
    mq_dma_all(q0, slot_d(0), seg_of(0), wave);
    mq_dma_all(q1, slot_d(1), seg_of(1), wave);
    mq_dma_all(q2, slot_d(2), seg_of(2), wave);
    __builtin_amdgcn_s_waitcnt(((2 * kQDma) & 15) | (7 << 4));  // slot 0 landed
    asm volatile("s_barrier" ::: "memory");
    Mx2Frag f0, f1;
    uint32_t sa[4], sw[2];
    mq_scales<NJ>(q0, o, sa, sw);
    mq_frags<NJ>(q0, o.la[0], o.lw[0], f0);
    for (int t = 0; t < T; t += 4) {
        mq_slot<NJ>(q0, q1, q3, slot_d(t + 3), seg_of(t + 3), o, wave, acc, f0, f1, sa, sw);
        mq_slot<NJ>(q1, q2, q0, slot_d(t + 4), seg_of(t + 4), o, wave, acc, f0, f1, sa, sw);
        mq_slot<NJ>(q2, q3, q1, slot_d(t + 5), seg_of(t + 5), o, wave, acc, f0, f1, sa, sw);
        mq_slot<NJ>(q3, q0, q2, slot_d(t + 6), seg_of(t + 6), o, wave, acc, f0, f1, sa, sw);
    }
    __builtin_amdgcn_s_waitcnt(0);  // the last (empty) copies landed
    __syncthreads();
    const int lane_e = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    mq_epilogue<OutT, NJ>(acc, q0, q1, q2, q3, g, m0, n0, wm, wn, lane_e, 64 * wave + lane_e);
}

template <bool AROW, bool WROW, int TN>
static void launch_seg_tiles(const MxGemmArgs &g, hipStream_t st)
{
    const int tiles = (int)(((g.M + MBM - 1) / MBM) * ((g.N + TN - 1) / TN));
    if (g.c_bf16)
        hipLaunchKernelGGL((k_mx_gemm_seg<__bf16, AROW, WROW, TN>), dim3(tiles), dim3(512), 0, st, g);
    else
        hipLaunchKernelGGL((k_mx_gemm_seg<float, AROW, WROW, TN>), dim3(tiles), dim3(512), 0, st, g);
}

// 256 x 256 tiles; when their last round would be at most half full and the
// columns of that round fit one round of 256 x 128 tiles, those columns go to a
// second launch of 256 x 128 tiles (M = 8192, N = 17408: eight rounds of large
// tiles over 16384 columns, then 256 tiles over the last 1024).
template <bool AROW, bool WROW>
static fp4_status launch_seg_layout(const MxGemmArgs &g, hipStream_t st)
{
    // 32-bit byte offsets and descriptor sizes
    if (g.K % kQK != 0 || g.M * (g.K / 2) >= (int64_t(1) << 31) || g.N * (g.K / 2) >= (int64_t(1) << 31))
        return FP4_ERR_SHAPE;
    MxGemmArgs a = g;
    a.w_row0 = 0;
    a.w_rows = g.N;
    const int64_t cus = device_cu_count();
    const int64_t tm = (g.M + MBM - 1) / MBM, tn = (g.N + MBN - 1) / MBN, tiles = tm * tn, rem = tiles % cus;
    if (tiles > cus && rem != 0 && rem <= cus / 2) {
        const int64_t n_split = tiles / cus * cus / tm * MBN;  // columns kept on large tiles
        if (n_split >= MBN && n_split < g.N && tm * ((g.N - n_split + 127) / 128) <= cus) {
            MxGemmArgs big = a;
            big.N = n_split;
            launch_seg_tiles<AROW, WROW, 256>(big, st);
            MxGemmArgs rest = a;
            rest.N = g.N - n_split;
            rest.w_row0 = n_split;
            rest.c = reinterpret_cast<uint8_t *>(g.c) + n_split * (g.c_bf16 ? 2 : 4);
            launch_seg_tiles<AROW, WROW, 128>(rest, st);
            return hipGetLastError() == hipSuccess ? FP4_OK : FP4_ERR_HIP;
        }
    }
    launch_seg_tiles<AROW, WROW, 256>(a, st);
    return hipGetLastError() == hipSuccess ? FP4_OK : FP4_ERR_HIP;
}

fp4_status launch_mxfp4_gemm_seg(const MxGemmArgs &g, hipStream_t st) { return launch_seg_layout<false, false>(g, st); }

fp4_status launch_mxfp4_gemm_seg_wrow(const MxGemmArgs &g, hipStream_t st)
{
    return launch_seg_layout<false, true>(g, st);
}


fp4_status launch_mxfp4_gemm(const MxGemmArgs &g, hipStream_t st)
{
    // the staged kernel addresses a matrix with 32-bit byte offsets
    if (g.K % kSK == 0 && g.M * (g.K / 2) < (int64_t(1) << 32) && g.N * (g.K / 2) < (int64_t(1) << 32)) {
        const int tiles = (int)(((g.M + MBM - 1) / MBM) * ((g.N + MBN - 1) / MBN));
        if (g.c_bf16)
            hipLaunchKernelGGL(k_mx_gemm_2s<__bf16>, dim3(tiles), dim3(512), 0, st, g);
        else
            hipLaunchKernelGGL(k_mx_gemm_2s<float>, dim3(tiles), dim3(512), 0, st, g);
        return hipGetLastError() == hipSuccess ? FP4_OK : FP4_ERR_HIP;
    }
    return launch_mx<false>(g, st);
}

}  // namespace fp4k
