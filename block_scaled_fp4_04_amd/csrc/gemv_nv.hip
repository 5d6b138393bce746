// gemv_nv.hip -- W4A16 decode GEMV (M <= 16) over NVFP4 weights kept in the
// decode layout, and the kernel that rewrites row-major NVFP4 weights into it.
//
// W4A16 (Unsloth Dynamic NVFP4 article, aixq.cc, section "Core difference:
// W4A4 vs W4A16"): 4-bit weights, 16-bit activations.  Decode multiplies a few
// activation rows by the whole weight, so the weight bytes (4.5 bits a value,
// "NVFP4" wiki, section "Technical principle") set the time; every design
// choice here serves streaming them at full HBM rate.
//
// Decode layout.  K is cut into 128-element segments; segment s of every row is
// 64 code bytes (row-major nibble order, element 2b in the low nibble of byte b)
// and 8 E4M3 scale bytes.  The layout stores segment-major:
//     codes_p[s][n][64]   (byte (s N + n) 64 + b = codes[n][64 s + b])
//     scales_p[s][n][8]   (byte (s N + n) 8 + b  = scales[n][8 s + b])
// so the 16 rows of an MFMA tile at one segment are 1 KiB of consecutive bytes:
// one 16-byte load per lane reads them with every 128-byte line whole, and any
// row offset works (a workgroup's row range needs no alignment).  The bytes and
// their count are those of the row-major form: only their order changes.
//
// GEMV.  A workgroup of 8 waves owns a run of consecutive rows, a whole number
// of 16-row tiles, with at most one workgroup per CU.  Wave w owns the K
// segments [S w, S w + S): its activation fragments are loaded once and stay in
// registers, and it walks the workgroup's 16-row tiles with loads for D - 1
// tiles in flight.  Lane (n, g) = (l % 16, l / 16) loads, per tile and segment,
// the 32 codes of row n at K 32 g .. 32 g + 31 and their 2 scale bytes; the
// codes feed four 16x16x32 bf16 MFMAs, MFMA j contracting K values
// 32 g + 8 j + [0, 8) of every lane group g (a permutation of K that the
// activation fragments share, so the sum is unchanged).  Each weight is widened
// exactly to E2M1 * E4M3 in bf16 (see dq8_bf16); accumulation is fp32.  The 8
// waves' partial tiles are added in LDS; the epilogue multiplies by the tensor
// scale.
// MXFP4 weights use the same decode layout with 4 E8M0 bytes per segment (one
// per 32-element block, lane group g's block): scales_p[s][n][4].  Their scales
// are powers of two, which the scaled E2M1 conversion applies exactly, so the MX
// variants need no separate scale multiply.
#include "device_common.h"
#include "internal.h"

namespace fp4k {

constexpr int kGvWaves = 8;
constexpr int kGvMaxT = 8;  // 16-row tiles per workgroup

// thread per (segment, row): 64 code bytes and 8 scale bytes (NVFP4) or 4 (MXFP4)
template <int SB>
__global__ __launch_bounds__(256) void k_pack_decode(const uint8_t *__restrict__ codes,
                                                         const uint8_t *__restrict__ scales, int N, int K,
                                                         uint8_t *__restrict__ cp, uint8_t *__restrict__ sp)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int nseg = K >> 7;
    if (idx >= (int64_t)N * nseg) return;
    const int s = (int)(idx / N), r = (int)(idx % N);
    const uint4 *src = reinterpret_cast<const uint4 *>(codes + (int64_t)r * (K / 2) + 64 * s);
    uint4 *dst = reinterpret_cast<uint4 *>(cp + idx * 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = src[i];
    if constexpr (SB == 8)
        *reinterpret_cast<uint2 *>(sp + idx * 8) = *reinterpret_cast<const uint2 *>(scales + (int64_t)r * (K / 16) + 8 * s);
    else
        *reinterpret_cast<uint32_t *>(sp + idx * 4) =
            *reinterpret_cast<const uint32_t *>(scales + (int64_t)r * (K / 32) + 4 * s);
}

// Buffer descriptor over `bytes` bytes at `base` (raw, byte-addressed; dword 3
// selects 32-bit data format).  A load whose offset is at or past `bytes`
// returns zeros and reads nothing, which is how rows past the workgroup's range,
// K segments a wave does not own and activation rows past M are skipped without
// any branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t gv_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

constexpr uint32_t kGvOut = 0x80000000u;  // an offset past every descriptor's size

template <int S>
struct GvTile {
    u32x4 c[S];     // 32 codes of row n, K 32 grp .. 32 grp + 31 of each segment
    uint32_t s[S];  // their two E4M3 scale bytes
};

// E2M1 x 4 (two code bytes, low nibble first) -> bf16 x 4, times the power of two
// in `scale`'s exponent field (1.0: unscaled); exact.
__device__ __forceinline__ bf16x4 e2m1x4_bf16(uint32_t w, int half, float scale = 1.0f)
{
    const bf16x2 lo = half ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2)
                           : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
    const bf16x2 hi = half ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3)
                           : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
    return bf16x4{lo[0], lo[1], hi[0], hi[1]};
}

// M4: M <= 4 variant.  Sixteen 4x4x4 bf16 MFMA blocks: block b = l / 4 multiplies
// activation rows 0..3 (lane 4 b + i supplies row i) by W rows 4 (b % 4) + j
// (lane 4 b + j, so lane l still owns W row l % 16) over K-quarter b / 4 of the
// segment, 4 K values per instruction.  The codes enter unscaled (E2M1 exactly
// in bf16); each NVFP4 block's four steps accumulate from zero and the partial is
// multiplied by the lane's E4M3 scale, so the scale costs 4 FMAs per 16 codes
// instead of a multiply per code.  The four K-quarters are summed across lanes
// at the end of the tile.
template <int S, int D, bool M4, int W, bool MX>
__global__ __launch_bounds__(64 * W, 1) void k_nv_gemv_dec(GemvArgs g)
{
    __shared__ f32x4 red[kGvMaxT][W][64];
    __shared__ __align__(16) uint16_t alds[M4 ? 4 * 1024 * S : 8];  // M4: A rows 0..3, K <= 1024 S
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, grp = lane >> 4;
    const int M = g.M, N = g.N;
    const int nseg = g.K >> 7;
    const int seg0 = wave * S;
    const int ns = max(0, min(S, nseg - seg0));  // this wave's segments
    const int r_lo = blockIdx.x * g.rows_per_wg;
    const int r_hi = min(r_lo + g.rows_per_wg, N);
    const int nt = (r_hi - r_lo + 15) >> 4;

    const __amdgpu_buffer_rsrc_t ra = gv_rsrc(g.a, (uint32_t)((int64_t)(M - 1) * g.lda * 2 + g.K * 2));
    const __amdgpu_buffer_rsrc_t rc = gv_rsrc(g.w_codes, (uint32_t)((int64_t)nseg * N * 64));
    constexpr int SB = MX ? 4 : 8;  // scale bytes per row and segment
    const __amdgpu_buffer_rsrc_t rs = gv_rsrc(g.w_scales, (uint32_t)((int64_t)nseg * N * SB));

    // byte offsets of this lane's codes / scales at tile 0, segment seg0 (kGvOut where skipped)
    uint32_t oc[S], os[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int64_t e = (int64_t)(seg0 + s) * N + r_lo + n;
        oc[s] = s < ns ? (uint32_t)(e * 64 + 16 * grp) : kGvOut;
        os[s] = s < ns ? (uint32_t)(e * SB + (MX ? 1 : 2) * grp) : kGvOut;
    }
    auto issue_seg = [&](int t, int s, GvTile<S> &b) {
        const bool ok = r_lo + 16 * t + n < r_hi;
        b.c[s] = __builtin_amdgcn_raw_buffer_load_b128(rc, (int)(ok ? oc[s] + 1024 * t : kGvOut), 0, 0);
        if constexpr (MX)
            b.s[s] = __builtin_amdgcn_raw_buffer_load_b8(rs, (int)(ok ? os[s] + 16 * SB * t : kGvOut), 0, 0);
        else
            b.s[s] = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)(ok ? os[s] + 16 * SB * t : kGvOut), 0, 0);
    };

    // activation fragments: A row n (M4: row l % 4; zero past M), K 128 (seg0 + s) + 32 grp + 8 j + [0, 8)
    const int arow = M4 ? (lane & 3) : n;
    bf16x8 af[S][4];
    GvTile<S> buf[D];
    if constexpr (M4) {
        // M <= 4: lanes 4 p + i (p = 0..3) need the same activation bytes, so the
        // workgroup stages A ([4][K] bf16, rows past M zero) in LDS once and every
        // wave reads its fragments from there.  The A loads go out first, then
        // the first tiles' weight loads, so waiting for A does not wait for them.
        constexpr int kAChunks = S;  // 16-byte chunks per thread: 4 * K / 8 <= 4 * 1024 S / 8 = 512 S
        const int cpr = g.K >> 3;    // chunks per row
        u32x4 ach[kAChunks];
#pragma unroll
        for (int c = 0; c < kAChunks; ++c) {
            const int idx = (int)threadIdx.x + 64 * W * c;
            const int row = idx / cpr, col = idx - row * cpr;
            const uint32_t off = (row < M && row < 4) ? (uint32_t)(((int64_t)row * g.lda + 8 * col) * 2) : kGvOut;
            ach[c] = __builtin_amdgcn_raw_buffer_load_b128(ra, (int)off, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < D - 1; ++k)
#pragma unroll
            for (int s = 0; s < S; ++s) issue_seg(k, s, buf[k]);
#pragma unroll
        for (int c = 0; c < kAChunks; ++c) {
            const int idx = (int)threadIdx.x + 64 * W * c;
            if (idx < 4 * cpr) *reinterpret_cast<u32x4 *>(alds + 8 * idx) = ach[c];
        }
        __builtin_amdgcn_s_waitcnt((0xF) | (0x3 << 14) | (7 << 4));  // lgkmcnt(0): this wave's A stores done
        asm volatile("s_barrier" ::: "memory");
#pragma unroll
        for (int s = 0; s < S; ++s)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                bf16x8 v = {};
                if (s < ns) v = *reinterpret_cast<const bf16x8 *>(alds + arow * g.K + 128 * (seg0 + s) + 32 * grp + 8 * j);
                af[s][j] = v;
            }
    } else {
        // loaded segment by segment between tile 0's weight loads so the first
        // math waits only for its own segment
#pragma unroll
        for (int s = 0; s < S; ++s) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t off = (s < ns && arow < M)
                    ? (uint32_t)(((int64_t)arow * g.lda + 128 * (seg0 + s) + 32 * grp + 8 * j) * 2) : kGvOut;
                const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(ra, (int)off, 0, 0);
                __builtin_memcpy(&af[s][j], &v, 16);
            }
            issue_seg(0, s, buf[0]);
        }
#pragma unroll
        for (int k = 1; k < D - 1; ++k)
#pragma unroll
            for (int s = 0; s < S; ++s) issue_seg(k, s, buf[k]);
    }

    typedef float f32x2 __attribute__((ext_vector_type(2)));
    // one segment of a tile, M <= 4 variant
    auto seg4 = [&](int s, const GvTile<S> &b, f32x4 &acc) {
        const f32x2 bs = __builtin_amdgcn_cvt_pk_f32_fp8((int)b.s[s], false);
        // the two NVFP4 blocks' MFMA chains interleaved, so each hides the other's latency
        f32x4 part[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                const int q = 4 * blk + st;  // K values 4 q .. 4 q + 3 of the lane's 32
                const bf16x8 a8 = af[s][q >> 1];
                const bf16x4 a4 = (q & 1) ? bf16x4{a8[4], a8[5], a8[6], a8[7]} : bf16x4{a8[0], a8[1], a8[2], a8[3]};
                part[blk] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a4, e2m1x4_bf16(b.c[s][q >> 1], q & 1), part[blk], 0, 0, 0);
            }
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(part[blk][i], bs[blk], acc[i]);
    };
    // one segment of a tile, 16x16x32 variant (two accumulator chains)
    // MXFP4, M <= 4: the lane's 32 codes are one MX block, whose power-of-two scale
    // the conversion applies exactly; two accumulator chains, no scale multiply
    auto seg4mx = [&](int s, const GvTile<S> &b, f32x4 &acc0, f32x4 &acc1) {
        const float sc = __uint_as_float(b.s[s] << 23);
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                const int q = 4 * blk + st;
                const bf16x8 a8 = af[s][q >> 1];
                const bf16x4 a4 = (q & 1) ? bf16x4{a8[4], a8[5], a8[6], a8[7]} : bf16x4{a8[0], a8[1], a8[2], a8[3]};
                f32x4 &acc = blk ? acc1 : acc0;
                acc = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a4, e2m1x4_bf16(b.c[s][q >> 1], q & 1, sc), acc, 0, 0, 0);
            }
    };
    auto seg16 = [&](int s, const GvTile<S> &b, f32x4 &acc0, f32x4 &acc1) {
        if constexpr (MX) {
            const float sc = __uint_as_float(b.s[s] << 23);
            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s][0], e2m1x8_bf16_pow2(b.c[s][0], sc), acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s][1], e2m1x8_bf16_pow2(b.c[s][1], sc), acc1, 0, 0, 0);
            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s][2], e2m1x8_bf16_pow2(b.c[s][2], sc), acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s][3], e2m1x8_bf16_pow2(b.c[s][3], sc), acc1, 0, 0, 0);
            return;
        }
        // the two E4M3 block scales of the lane's 32 codes (OCP E4M3FN conversion)
        const f32x2 bs = __builtin_amdgcn_cvt_pk_f32_fp8((int)b.s[s], false);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s][0], as_bf16x8(dq8_bf16(b.c[s][0], bs[0])), acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s][1], as_bf16x8(dq8_bf16(b.c[s][1], bs[0])), acc1, 0, 0, 0);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s][2], as_bf16x8(dq8_bf16(b.c[s][2], bs[1])), acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[s][3], as_bf16x8(dq8_bf16(b.c[s][3], bs[1])), acc1, 0, 0, 0);
    };

    // D tiles in flight.  The tile loop is unrolled completely, so every buffer is
    // a fixed register set and no load in flight crosses a loop back edge.  The
    // loads of tile t + D - 1 are spread over tile t's segments, one segment's
    // loads before each segment's math, so the wave keeps loads in flight while it
    // computes; loads for tiles at or past nt read nothing.
#pragma unroll
    for (int t = 0; t < kGvMaxT; ++t) {
        if (t < nt) {
            f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll
            for (int s = 0; s < S; ++s) {
                if (t + D - 1 < kGvMaxT) issue_seg(t + D - 1, s, buf[(t + D - 1) % D]);
                __builtin_amdgcn_sched_barrier(0);
                if (M4 && MX)
                    seg4mx(s, buf[t % D], acc0, acc1);
                else if (M4)
                    seg4(s, buf[t % D], acc0);
                else
                    seg16(s, buf[t % D], acc0, acc1);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (M4) {
                if (MX) acc0 += acc1;
                // sum the four K-quarters (lanes l, l ^ 16, l ^ 32, l ^ 48)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc0[i] += __shfl_xor(acc0[i], 16);
                    acc0[i] += __shfl_xor(acc0[i], 32);
                }
                red[t][wave][lane] = acc0;
            } else {
                red[t][wave][lane] = acc0 + acc1;
            }
        }
    }
    __syncthreads();

    // wave w finishes tile w: lane (n, grp) holds rows 4 grp + i of output column
    // r_lo + 16 w + n (M4: lanes with grp = 0 hold rows 0..3)
    if (wave < nt) {
        f32x4 sum = red[wave][0][lane];
#pragma unroll
        for (int w = 1; w < W; ++w) sum += red[wave][w][lane];
        const float ts = MX ? 1.f : *g.w_tscale;  // MXFP4 has no tensor scale
        const int col = r_lo + 16 * wave + n;
        if (col < r_hi) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * grp + i;
                if (m < M) {
                    const float o = sum[i] * ts;
                    if (g.c_bf16)
                        reinterpret_cast<__bf16 *>(g.c)[(int64_t)m * g.ldc + col] = (__bf16)o;
                    else
                        reinterpret_cast<float *>(g.c)[(int64_t)m * g.ldc + col] = o;
                }
            }
        }
    }
}

fp4_status launch_pack_decode(const uint8_t *codes, const uint8_t *scales, int64_t N, int64_t K,
                              uint8_t *codes_p, uint8_t *scales_p, bool mx, hipStream_t st)
{
    const int64_t threads = N * (K / 128);
    if (threads == 0) return FP4_OK;
    const dim3 grid((unsigned)((threads + 255) / 256));
    if (mx)
        hipLaunchKernelGGL(k_pack_decode<4>, grid, dim3(256), 0, st, codes, scales, (int)N, (int)K, codes_p, scales_p);
    else
        hipLaunchKernelGGL(k_pack_decode<8>, grid, dim3(256), 0, st, codes, scales, (int)N, (int)K, codes_p, scales_p);
    return hipGetLastError() == hipSuccess ? FP4_OK : FP4_ERR_HIP;
}

template <int S, bool MX>
static void launch_gemv(const GemvArgs &g, unsigned grid, hipStream_t st)
{
    constexpr int D = S <= 5 ? 3 : 2;  // tiles in flight, bounded by registers
    // the M <= 4 variant's extra registers do not fit beside 8 segments' fragments
    if constexpr (S < 8) {
        if (g.M <= 4) {
            hipLaunchKernelGGL((k_nv_gemv_dec<S, D, true, kGvWaves, MX>), dim3(grid), dim3(64 * kGvWaves), 0, st, g);
            return;
        }
    }
    hipLaunchKernelGGL((k_nv_gemv_dec<S, D, false, kGvWaves, MX>), dim3(grid), dim3(64 * kGvWaves), 0, st, g);
}

template <int S>
static void launch_gemv_fmt(const GemvArgs &g, unsigned grid, hipStream_t st)
{
    if (g.mx) launch_gemv<S, true>(g, grid, st);
    else launch_gemv<S, false>(g, grid, st);
}

int device_cu_count()
{
    static int cache[64] = {0};  // per device; benign race: every writer stores the same value
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cache[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

fp4_status launch_gemv_decode(GemvArgs g, hipStream_t st)
{
    const int nseg = g.K / 128;
    const int S = (nseg + kGvWaves - 1) / kGvWaves;
    // whole 16-row tiles per workgroup, all workgroups in one round (at most one
    // per CU): a workgroup's last tile is multiplied in full whether or not its
    // rows exist, and that math is not hidden under the loads, so fewer, full
    // workgroups beat one per CU with a partial last tile (N = 17408: 218
    // workgroups of 80 rows run faster than 256 of 68).  More workgroups than
    // CUs only when a CU's share would exceed kGvMaxT tiles.
    const int64_t tiles = (g.N + 15) / 16, cus = device_cu_count();
    const int64_t per = std::min<int64_t>((tiles + cus - 1) / cus, kGvMaxT);
    const int64_t R = 16 * per;
    const int64_t G = (g.N + R - 1) / R;
    g.rows_per_wg = (int)R;
    switch (S) {
    case 1: launch_gemv_fmt<1>(g, (unsigned)G, st); break;
    case 2: launch_gemv_fmt<2>(g, (unsigned)G, st); break;
    case 3: launch_gemv_fmt<3>(g, (unsigned)G, st); break;
    case 4: launch_gemv_fmt<4>(g, (unsigned)G, st); break;
    case 5: launch_gemv_fmt<5>(g, (unsigned)G, st); break;
    case 6: launch_gemv_fmt<6>(g, (unsigned)G, st); break;
    case 7: launch_gemv_fmt<7>(g, (unsigned)G, st); break;
    case 8: launch_gemv_fmt<8>(g, (unsigned)G, st); break;
    default: return FP4_ERR_SHAPE;
    }
    return hipGetLastError() == hipSuccess ? FP4_OK : FP4_ERR_HIP;
}

}  // namespace fp4k
