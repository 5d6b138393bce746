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
// GEMV.  One workgroup of 8 waves per CU owns ceil(N / G) consecutive rows
// (G workgroups), so every CU streams the same weight bytes.  Wave w owns the K
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
#include "device_common.h"
#include "internal.h"

namespace fp4k {

constexpr int kGvWaves = 8;
constexpr int kGvMaxT = 8;  // 16-row tiles per workgroup

// thread per (segment, row): 64 code bytes and 8 scale bytes
__global__ __launch_bounds__(256) void k_nv_pack_decode(const uint8_t *__restrict__ codes,
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
    *reinterpret_cast<uint2 *>(sp + idx * 8) =
        *reinterpret_cast<const uint2 *>(scales + (int64_t)r * (K / 16) + 8 * s);
}

template <int S, int D>
__global__ __launch_bounds__(512, 1) void k_nv_gemv_dec(GemvArgs g)
{
    __shared__ f32x4 red[kGvMaxT][kGvWaves][64];
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

    // activation fragments: A row n (zero past M), K 128 (seg0 + s) + 32 grp + 8 j + [0, 8)
    bf16x8 af[S][4];
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            bf16x8 v = {};
            if (s < ns && n < M)
                v = *reinterpret_cast<const bf16x8 *>(g.a + (int64_t)n * g.lda + 128 * (seg0 + s) + 32 * grp + 8 * j);
            af[s][j] = v;
        }

    u32x4 wc[D][S];
    uint32_t wsc[D][S];
    auto issue = [&](int t, int b) {
        const int row = r_lo + 16 * t + n;
        const bool ok = row < r_hi;
#pragma unroll
        for (int s = 0; s < S; ++s) {
            u32x4 c = {0u, 0u, 0u, 0u};
            uint32_t sc = 0;
            if (s < ns && ok) {
                const int64_t e = (int64_t)(seg0 + s) * N + row;
                c = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(g.w_codes + e * 64 + 16 * grp));
                sc = *reinterpret_cast<const uint16_t *>(g.w_scales + e * 8 + 2 * grp);
            }
            wc[b][s] = c;
            wsc[b][s] = sc;
        }
    };

#pragma unroll
    for (int t = 0; t < D - 1; ++t)
        if (t < nt) issue(t, t);
#pragma unroll
    for (int t = 0; t < kGvMaxT; ++t) {
        if (t < nt) {
            if (t + D - 1 < nt) issue(t + D - 1, (t + D - 1) % D);
            const int b = t % D;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < S; ++s) {
                if (s < ns) {
                    // the two E4M3 block scales of the lane's 32 codes (OCP E4M3FN conversion)
                    typedef float f32x2 __attribute__((ext_vector_type(2)));
                    const f32x2 bs = __builtin_amdgcn_cvt_pk_f32_fp8((int)wsc[b][s], false);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            af[s][j], as_bf16x8(dq8_bf16(wc[b][s][j], j < 2 ? bs[0] : bs[1])), acc, 0, 0, 0);
                }
            }
            red[t][wave][lane] = acc;
        }
    }
    __syncthreads();

    // wave w finishes tile w: lane (n, grp) holds rows 4 grp + i of output column r_lo + 16 w + n
    if (wave < nt) {
        f32x4 sum = red[wave][0][lane];
#pragma unroll
        for (int w = 1; w < kGvWaves; ++w) sum += red[wave][w][lane];
        const float ts = *g.w_tscale;
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

fp4_status launch_nvfp4_pack_decode(const uint8_t *codes, const uint8_t *scales, int64_t N, int64_t K,
                                    uint8_t *codes_p, uint8_t *scales_p, hipStream_t st)
{
    const int64_t threads = N * (K / 128);
    if (threads == 0) return FP4_OK;
    hipLaunchKernelGGL(k_nv_pack_decode, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, codes, scales,
                       (int)N, (int)K, codes_p, scales_p);
    return hipGetLastError() == hipSuccess ? FP4_OK : FP4_ERR_HIP;
}

template <int S>
static void launch_gemv(const GemvArgs &g, unsigned grid, hipStream_t st)
{
    constexpr int D = S <= 5 ? 3 : 2;  // tiles in flight, bounded by registers
    hipLaunchKernelGGL((k_nv_gemv_dec<S, D>), dim3(grid), dim3(64 * kGvWaves), 0, st, g);
}

static int cu_count()
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

fp4_status launch_nvfp4_gemv_decode(GemvArgs g, hipStream_t st)
{
    const int nseg = g.K / 128;
    const int S = (nseg + kGvWaves - 1) / kGvWaves;
    // one workgroup per CU with equal row counts; more workgroups only when a
    // CU's share exceeds kGvMaxT tiles
    int64_t G = std::min<int64_t>(cu_count(), (g.N + 15) / 16);
    int64_t R = (g.N + G - 1) / G;
    if (R > 16 * kGvMaxT) {
        G = (g.N + 16 * kGvMaxT - 1) / (16 * kGvMaxT);
        R = (g.N + G - 1) / G;
    }
    G = (g.N + R - 1) / R;
    g.rows_per_wg = (int)R;
    switch (S) {
    case 1: launch_gemv<1>(g, (unsigned)G, st); break;
    case 2: launch_gemv<2>(g, (unsigned)G, st); break;
    case 3: launch_gemv<3>(g, (unsigned)G, st); break;
    case 4: launch_gemv<4>(g, (unsigned)G, st); break;
    case 5: launch_gemv<5>(g, (unsigned)G, st); break;
    case 6: launch_gemv<6>(g, (unsigned)G, st); break;
    case 7: launch_gemv<7>(g, (unsigned)G, st); break;
    case 8: launch_gemv<8>(g, (unsigned)G, st); break;
    default: return FP4_ERR_SHAPE;
    }
    return hipGetLastError() == hipSuccess ? FP4_OK : FP4_ERR_HIP;
}

}  // namespace fp4k
