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
// segments [S w, S w + S) of all the workgroup's tiles (the walk is described
// above k_nv_gemv_dec).  Lane (n, g) = (l % 16, l / 16) loads, per tile and segment,
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

// s_waitcnt vmcnt(N): wait until at most N vector-memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void nv_wait_vm_gv()
{
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// the same for a count that is a compile-time constant only once the walk is
// unrolled (the switch then folds to one wait)
__device__ __forceinline__ void nv_wait_vm_gv_n(int n)
{
    switch (n) {
    case 0: nv_wait_vm_gv<0>(); break;
    case 1: nv_wait_vm_gv<1>(); break;
    case 2: nv_wait_vm_gv<2>(); break;
    case 3: nv_wait_vm_gv<3>(); break;
    case 4: nv_wait_vm_gv<4>(); break;
    case 5: nv_wait_vm_gv<5>(); break;
    case 6: nv_wait_vm_gv<6>(); break;
    case 7: nv_wait_vm_gv<7>(); break;
    default: nv_wait_vm_gv<8>(); break;
    }
}

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

// Work order.  A wave owns the K segments seg0 .. seg0 + S - 1 and the
// workgroup's NT tiles; it walks them segment-major, (s, t) = (0, 0), (0, 1),
// ..., (1, 0), ..., with one accumulator set per tile, so it needs one segment's
// activation fragments at a time (the next segment's are fetched while the
// current one is used) and the 16 x 16 variant's 160 KiB of activations per CU
// arrive spread over the kernel instead of all before the first product.  The
// weight loads run D units (tile and segment) ahead.  S and NT are compile-time,
// so every buffer index is fixed and the whole walk is one basic block per unit.
//
// M4: M <= 4 variant.  Sixteen 4x4x4 bf16 MFMA blocks: block b = l / 4 multiplies
// activation rows 0..3 (lane 4 b + i supplies row i) by W rows 4 (b % 4) + j
// (lane 4 b + j, so lane l still owns W row l % 16) over K-quarter b / 4 of the
// segment, 4 K values per instruction.  The codes enter unscaled (E2M1 exactly
// in bf16); each NVFP4 block's four steps accumulate from zero and the partial is
// multiplied by the lane's E4M3 scale, so the scale costs 4 FMAs per 16 codes
// instead of a multiply per code.  The four K-quarters are summed across lanes
// at the end (lane-swap instructions, no LDS).  The activation rows (4 x K bf16)
// are staged in LDS once per workgroup: the lanes 4 p + i of a wave all need
// row i.  (Loading each wave's fragments from memory instead, with no
// workgroup barrier, was about 1 us slower at M = 4: 20 more memory
// instructions per wave, 4 lanes reading each address.)
// M1 (with M4): exactly one activation row; of the four rows the 4x4x4 blocks
// produce only row 0 is scaled, reduced and stored.
// CH: K spans more than one chunk (K > 1024 S).  Kept a template flag: as a
// runtime loop even of one pass, the chunk loop made the compiler carry the
// accumulators through a loop with copies (2-4% slower at K = 5120).
template <int S, int NT, bool M4, bool MX, bool M1 = false, bool CH = false>
__global__ __launch_bounds__(64 * kGvWaves, 1) void k_nv_gemv_dec(GemvArgs g)
{
    constexpr int W = kGvWaves;
    constexpr int D = M4 ? 8 : 4;  // units (tile, segment) of weight loads in flight (measured best: 3..8 tried)
    __shared__ f32x4 red[NT][W][64];
    __shared__ __align__(16) uint16_t alds[M4 ? 4 * 1024 * S : 8];  // M4: A rows 0..3, K <= 1024 S
    __shared__ __align__(16) uint8_t a16[M4 ? 16 : W * 2 * 4096];    // M > 4: per wave, two segments of A
    __shared__ __align__(16) uint8_t sclds[W][M4 ? 16 : 1024];       // M > 4, per wave: one segment's block scales
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, grp = lane >> 4;
    const int M = g.M, N = g.N;
    const int nseg = g.K >> 7;
    // K runs in chunks of 8 S segments (one when K <= 1024 S): the wave owns
    // segments seg0 .. seg0 + ns - 1 of the current chunk, which starts at segment
    // segb and spans wch K elements
    const int nch = (nseg + W * S - 1) / (W * S);
    int segb = 0, seg0 = wave * S, ns = max(0, min(S, nseg - seg0)), wch = min(g.K, 1024 * S);
    const int r_lo = blockIdx.x * g.rows_per_wg;
    const int r_hi = min(r_lo + g.rows_per_wg, N);
    const int nt = (r_hi - r_lo + 15) >> 4;      // <= NT

    const __amdgpu_buffer_rsrc_t ra = gv_rsrc(g.a, (uint32_t)((int64_t)(M - 1) * g.lda * 2 + g.K * 2));
    const __amdgpu_buffer_rsrc_t rc = gv_rsrc(g.w_codes, (uint32_t)((int64_t)nseg * N * 64));
    constexpr int SB = MX ? 4 : 8;  // scale bytes per row and segment
    const __amdgpu_buffer_rsrc_t rs = gv_rsrc(g.w_scales, (uint32_t)((int64_t)nseg * N * SB));
    // the tensor scale is read now, not in the epilogue, where its load would wait
    // behind the weight stream
    const float ts = MX ? 1.0f : *g.w_tscale;

    // unit u = (segment u / NT, tile u % NT): the lane's 32 codes (row n, K 32 grp ..)
    // and their scale byte(s); rows past the workgroup's range and segments the
    // wave does not own read nothing
    // The lane's code byte offset within a segment, per tile (fixed for the whole
    // walk: rows past the range get kGvOut), and the segment's start as the scalar
    // offset; a segment the wave does not own goes through size-0 descriptors.
    // So a unit's load takes no vector arithmetic.  Offsets stay below 2^32: the
    // segment starts are below the codes' size (< 2^31, checked on the host).
    uint32_t vo_c[NT], vo_s[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int row = r_lo + 16 * t + n;
        vo_c[t] = row < r_hi ? (uint32_t)row * 64u + 16u * grp : kGvOut;
        vo_s[t] = row < r_hi ? (uint32_t)row * SB + (MX ? 1u : 2u) * grp : kGvOut;
    }
    const __amdgpu_buffer_rsrc_t rc0 = gv_rsrc(g.w_codes, 0), rs0 = gv_rsrc(g.w_scales, 0);
    // M <= 4: a unit loads its codes and its lane's scale byte(s).  M > 4 takes the
    // scales per segment instead (below).  Weight loads carry the non-temporal
    // hint (cache policy 2): every weight byte is read once per call, and so does
    // not displace what is reused, such as the activations every workgroup reads
    // (N = 17408, K = 5120, weights streamed from HBM: 4-7% faster; slower only
    // when all the weights a loop cycles through fit in the 256 MB Infinity Cache).
    auto issue = [&](int u, u32x4 &c, uint32_t &sc) {
        const int s = u / NT, t = u % NT;
        const bool own = s < ns;  // wave-uniform
        const int seg = own ? seg0 + s : 0;
        c = __builtin_amdgcn_raw_buffer_load_b128(own ? rc : rc0, (int)vo_c[t], seg * N * 64, 2);
        if constexpr (M4) {
            if constexpr (MX)
                sc = __builtin_amdgcn_raw_buffer_load_b8(own ? rs : rs0, (int)vo_s[t], seg * N * SB, 2);
            else
                sc = __builtin_amdgcn_raw_buffer_load_b16(own ? rs : rs0, (int)vo_s[t], seg * N * SB, 2);
        }
    };
    // M > 4: block scales per segment.  The workgroup's rows are consecutive, so one
    // segment's scale bytes of all its tiles are one run of 16 NT SB bytes (640 for
    // NVFP4 with 5 tiles): one 16-byte load per lane fetches them (lanes past the
    // run read nothing), the wave parks them in its LDS slot, and each unit reads
    // its lane's byte(s) back.  This takes one load instruction per unit off the
    // address unit (13.5 -> 13.1 us at M = 16); at M <= 4, whose units are shorter,
    // the per-unit LDS read cost more than it saved (11.0 -> 11.3 us at M = 1).
    constexpr int kScLanes = (16 * NT * SB + 15) / 16;
    auto sc_load = [&](int s) -> u32x4 {
        const bool own = s < ns;
        const int seg = own ? seg0 + s : 0;
        const uint32_t off = lane < kScLanes ? 16u * lane : kGvOut;
        return __builtin_amdgcn_raw_buffer_load_b128(own ? rs : rs0, (int)off, (seg * N + r_lo) * SB, 2);
    };
    auto sc_park = [&](const u32x4 &v) { *reinterpret_cast<u32x4 *>(&sclds[wave][16 * lane]) = v; };
    auto sc_read = [&](int t) -> uint32_t {
        const int b = (16 * t + n) * SB + (MX ? 1 : 2) * grp;
        if constexpr (MX)
            return sclds[wave][b];
        else
            return *reinterpret_cast<const uint16_t *>(&sclds[wave][b]);
    };
    // activation fragments of segment s: A row arow (zero past M), K 128 (seg0 + s) + 32 grp + 8 j + [0, 8).
    // M <= 4 reads them from the workgroup's staged rows.  M > 4 copies each
    // segment's 16 rows x 128 K (4 KiB) into one of the wave's two LDS buffers by
    // DMA first: copy i covers rows 4 i .. 4 i + 3 as whole 256-byte row pieces
    // (lane L lands in row 4 i + L / 16, slot L % 16 and fetches the row's 16-byte
    // chunk slot ^ row), 8 cache lines per copy where a fragment load straight from
    // memory touches 32; the chunk swizzle lets each 16-lane group of a fragment
    // read hit 16 different bank groups.
    const int arow = M4 ? (lane & 3) : n;
    // A segment the wave does not own reads a valid one and selects zeros, with
    // no branch: the walk then has none at all, and the accumulators keep their
    // registers from unit to unit (around a branch the compiler copied them whole).
    auto frags = [&](int s, bf16x8 (&dst)[4]) {
        const bool own = s < ns;  // wave-uniform
        const int sg = min(seg0 + s, nseg - 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bf16x8 v = *reinterpret_cast<const bf16x8 *>(alds + arow * wch + 128 * (sg - segb) + 32 * grp + 8 * j);
            dst[j] = own ? v : bf16x8{};
        }
    };
    typedef __attribute__((address_space(3))) void gv_lds_void;
    auto a_dma = [&](int s, int b) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * i + (lane >> 4), slot = lane & 15, ch = slot ^ r;
            const uint32_t off =
                (s < ns && r < M) ? (uint32_t)(((int64_t)r * g.lda + 128 * (seg0 + s)) * 2 + 16 * ch) : kGvOut;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (gv_lds_void *)(a16 + 8192 * wave + 4096 * b + 1024 * i), 16,
                                                     (int)off, 0, 0, 0);
        }
    };
    auto frags16 = [&](int b, bf16x8 (&dst)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            dst[j] = *reinterpret_cast<const bf16x8 *>(a16 + 8192 * wave + 4096 * b + 256 * n + 16 * ((4 * grp + j) ^ n));
    };

    typedef float f32x2 __attribute__((ext_vector_type(2)));
    f32x4 acc[NT][2];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t][0] = acc[t][1] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 bc[D];
    uint32_t bsc[D];  // M <= 4: the units' scale byte(s)
    u32x4 scv;        // M > 4: the next segment's scale run, in flight
    for (int ch = 0; ch < (CH ? nch : 1); ++ch) {
    segb = ch * W * S;
    seg0 = segb + wave * S;
    ns = max(0, min(S, nseg - seg0));
    wch = min(1024 * S, g.K - 128 * segb);
    if constexpr (M4) {
        // the A loads go out first, then the first units' weight loads, so waiting
        // for A does not wait for them; a later chunk overwrites the staged rows
        // only once every wave has read the previous chunk's
        if (ch > 0) __syncthreads();
        const int cpr = wch >> 3;  // 16-byte chunks per row; 4 cpr <= 512 S = 64 W S / 8 chunks
        u32x4 ach[S];
#pragma unroll
        for (int c = 0; c < S; ++c) {
            const int idx = (int)threadIdx.x + 64 * W * c;
            const int row = idx / cpr, col = idx - row * cpr;
            const uint32_t off =
                (row < M && row < 4) ? (uint32_t)(((int64_t)row * g.lda + 128 * segb + 8 * col) * 2) : kGvOut;
            ach[c] = __builtin_amdgcn_raw_buffer_load_b128(ra, (int)off, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < D - 1; ++k)
            if (k < S * NT) issue(k, bc[k], bsc[k]);
#pragma unroll
        for (int c = 0; c < S; ++c) {
            const int idx = (int)threadIdx.x + 64 * W * c;
            if (idx < 4 * cpr) *reinterpret_cast<u32x4 *>(alds + 8 * idx) = ach[c];
        }
        __builtin_amdgcn_s_waitcnt((0xF) | (0x3 << 14) | (7 << 4));  // lgkmcnt(0): this wave's A stores done
        asm volatile("s_barrier" ::: "memory");
    }
    bf16x8 af[2][4];
    if constexpr (M4) {
        frags(0, af[0]);
    } else {
        // the scale run goes out before the copy, in a scheduling region of its
        // own, so that only code loads follow the copy (the wait counts below)
        scv = sc_load(0);
        __builtin_amdgcn_sched_barrier(0);
        a_dma(0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < D - 1; ++k)
            if (k < S * NT) issue(k, bc[k], bsc[k]);
        __builtin_amdgcn_sched_barrier(0);
    }


    // one unit: the lane's 32 codes c with scale byte(s) sc against fragments a
    auto unit = [&](const bf16x8 (&a)[4], const u32x4 &c, uint32_t sc, f32x4 &acc0, f32x4 &acc1) {
        if constexpr (M4) {
            const float msc = MX ? __uint_as_float(sc << 23) : 1.0f;  // MXFP4: the block's power of two
            f32x4 part[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
            // the two accumulation chains interleaved, so each hides the other's latency
#pragma unroll
            for (int st = 0; st < 4; ++st)
#pragma unroll
                for (int blk = 0; blk < 2; ++blk) {
                    const int q = 4 * blk + st;  // K values 4 q .. 4 q + 3 of the lane's 32
                    const bf16x8 a8 = a[q >> 1];
                    const bf16x4 a4 = (q & 1) ? bf16x4{a8[4], a8[5], a8[6], a8[7]} : bf16x4{a8[0], a8[1], a8[2], a8[3]};
                    f32x4 &dst = MX ? (blk ? acc1 : acc0) : part[blk];
                    dst = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a4, e2m1x4_bf16(c[q >> 1], q & 1, msc), dst, 0, 0, 0);
                }
            if constexpr (!MX) {
                // each NVFP4 block's partial times its E4M3 scale
                const f32x2 bs = __builtin_amdgcn_cvt_pk_f32_fp8((int)sc, false);
#pragma unroll
                for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                    for (int i = 0; i < (M1 ? 1 : 4); ++i) acc0[i] = __builtin_fmaf(part[blk][i], bs[blk], acc0[i]);
                // the sums are formed here, in the unit: left free, the compiler
                // deferred these FMAs to later units and kept every unit's
                // partials live (about 8 more registers per unit, and spills)
#pragma unroll
                for (int i = 0; i < (M1 ? 1 : 4); ++i) asm volatile("" : "+v"(acc0[i]));
            }
        } else if constexpr (MX) {
            const float msc = __uint_as_float(sc << 23);
            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], e2m1x8_bf16_pow2(c[0], msc), acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1], e2m1x8_bf16_pow2(c[1], msc), acc1, 0, 0, 0);
            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[2], e2m1x8_bf16_pow2(c[2], msc), acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[3], e2m1x8_bf16_pow2(c[3], msc), acc1, 0, 0, 0);
        } else {
            // the two E4M3 block scales of the lane's 32 codes (OCP E4M3FN conversion)
            const f32x2 bs = __builtin_amdgcn_cvt_pk_f32_fp8((int)sc, false);
            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], as_bf16x8(dq8_bf16(c[0], bs[0])), acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1], as_bf16x8(dq8_bf16(c[1], bs[0])), acc1, 0, 0, 0);
            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[2], as_bf16x8(dq8_bf16(c[2], bs[1])), acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[3], as_bf16x8(dq8_bf16(c[3], bs[1])), acc1, 0, 0, 0);
        }
    };

    // the walk: fully unrolled and free of branches, so every buffer is a fixed
    // register set and no load in flight crosses a loop back edge.  Units of tiles
    // at or past nt (rows past the range) and of segments the wave does not own
    // read nothing and multiply zero codes: their sums are zero or never stored.
#pragma unroll
    for (int s = 0; s < S; ++s) {
        // The two waves of a SIMD (w and w + 4) take turns at issue priority,
        // segment by segment.  Issue goes to the older wave first at equal
        // priority, and without the turns waves 0-3 ended their walks about
        // 1 us before waves 4-7 (shader timestamps), which then streamed alone;
        // with them the walks end within 0.15-0.65 us of each other (0.5-1%
        // faster at N = 17408, up to 3% at N = 16384, M = 16).
        if (((s + (wave >> 2)) & 1) != 0)
            __builtin_amdgcn_s_setprio(1);
        else
            __builtin_amdgcn_s_setprio(0);
        if constexpr (M4) {
            if (s + 1 < S) frags(s + 1, af[(s + 1) & 1]);
        } else {
            // segment s's copy is older than every load issued after it: the code
            // loads of the units the walk looks ahead to, D - 1 before segment 0 and
            // NT per segment, fewer at the end of the walk, where units past the last
            // are not loaded (the compiler would drop loads whose data go unused,
            // and the counts must be exact; the next segment's scale run goes out
            // before its copy)
            const int ahead = s == 0 ? min(D - 1, S * NT) : max(0, min(NT, S * NT - ((s - 1) * NT + D - 1)));
            nv_wait_vm_gv_n(ahead);
            __builtin_amdgcn_sched_barrier(0);
            frags16(s & 1, af[s & 1]);
            // segment s's scales to the LDS slot (the wave's reads of segment s - 1's
            // are older: a wave's LDS operations complete in order), the next run out
            sc_park(scv);
            if (s + 1 < S) scv = sc_load(s + 1);
            __builtin_amdgcn_sched_barrier(0);
            if (s + 1 < S) a_dma(s + 1, (s + 1) & 1);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int u = s * NT + t;
            if (u + D - 1 < S * NT) issue(u + D - 1, bc[(u + D - 1) % D], bsc[(u + D - 1) % D]);
            __builtin_amdgcn_sched_barrier(0);
            {
                uint32_t sc;
                if constexpr (M4)
                    sc = bsc[u % D];
                else
                    sc = sc_read(t);
                unit(af[s & 1], bc[u % D], sc, acc[t][0], acc[t][1]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    }  // chunks

#pragma unroll
    for (int t = 0; t < NT; ++t) {
        if (t < nt) {
            f32x4 v = M4 && !MX ? acc[t][0] : acc[t][0] + acc[t][1];
            if constexpr (M4) {
                // sum the four K-quarters (lanes l, l ^ 16, l ^ 32, l ^ 48): each swap
                // returns the value with its rows of 16 (or halves of 32) exchanged,
                // and the two results add up to lane l's and its partner's
#pragma unroll
                for (int i = 0; i < (M1 ? 1 : 4); ++i) {
                    const auto h16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[i]),
                                                                      false, false);
                    v[i] = __uint_as_float(h16[0]) + __uint_as_float(h16[1]);
                    const auto h32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), __float_as_uint(v[i]),
                                                                      false, false);
                    v[i] = __uint_as_float(h32[0]) + __uint_as_float(h32[1]);
                }
            }
            red[t][wave][lane] = v;
        }
    }
    __syncthreads();

    // wave w finishes tile w: lane (n, grp) holds rows 4 grp + i of output column
    // r_lo + 16 w + n (M4: lanes with grp = 0 hold rows 0..3)
    if (wave < nt) {
        f32x4 sum = red[wave][0][lane];
#pragma unroll
        for (int w = 1; w < W; ++w) sum += red[wave][w][lane];
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

template <int S, int NT, bool MX, bool CH>
static void launch_gemv_ch(const GemvArgs &g, unsigned grid, hipStream_t st)
{
    if (g.M == 1 && !MX)
        hipLaunchKernelGGL((k_nv_gemv_dec<S, NT, true, MX, true, CH>), dim3(grid), dim3(64 * kGvWaves), 0, st, g);
    else if (g.M <= 4)
        hipLaunchKernelGGL((k_nv_gemv_dec<S, NT, true, MX, false, CH>), dim3(grid), dim3(64 * kGvWaves), 0, st, g);
    else
        hipLaunchKernelGGL((k_nv_gemv_dec<S, NT, false, MX, false, CH>), dim3(grid), dim3(64 * kGvWaves), 0, st, g);
}

// more than one chunk only arises with S >= 5 (K > 8192 gives at least 65
// segments over chunks of 8 S), so only those S have the chunked form
template <int S, int NT, bool MX>
static void launch_gemv(const GemvArgs &g, unsigned grid, hipStream_t st)
{
    if constexpr (S >= 5) {
        if (g.K > 1024 * S) {
            launch_gemv_ch<S, NT, MX, true>(g, grid, st);
            return;
        }
    }
    launch_gemv_ch<S, NT, MX, false>(g, grid, st);
}

template <int S, int NT>
static void launch_gemv_fmt(const GemvArgs &g, unsigned grid, hipStream_t st)
{
    if (g.mx) launch_gemv<S, NT, true>(g, grid, st);
    else launch_gemv<S, NT, false>(g, grid, st);
}

template <int S>
static void launch_gemv_nt(const GemvArgs &g, int nt, unsigned grid, hipStream_t st)
{
    switch (nt) {
    case 1: launch_gemv_fmt<S, 1>(g, grid, st); break;
    case 2: launch_gemv_fmt<S, 2>(g, grid, st); break;
    case 3: launch_gemv_fmt<S, 3>(g, grid, st); break;
    case 4: launch_gemv_fmt<S, 4>(g, grid, st); break;
    case 5: launch_gemv_fmt<S, 5>(g, grid, st); break;
    case 6: launch_gemv_fmt<S, 6>(g, grid, st); break;
    case 7: launch_gemv_fmt<S, 7>(g, grid, st); break;
    default: launch_gemv_fmt<S, 8>(g, grid, st); break;
    }
}

int device_cu_count()
{
    static std::atomic<int> cache[64];  // per device; 0 until first asked (zero-initialized: static storage)
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (!n) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev].store(n, std::memory_order_relaxed);  // every writer stores the same value
    }
    return n;
}

fp4_status launch_gemv_decode(GemvArgs g, hipStream_t st)
{
    const int nseg = g.K / 128;
    // segments per wave and chunk: K beyond 1024 * 8 runs in chunks of 8 S
    // segments, S chosen so the chunks come out as even as they go
    const int nch = (nseg + 8 * kGvWaves - 1) / (8 * kGvWaves);
    const int S = (nseg + kGvWaves * nch - 1) / (kGvWaves * nch);
    if (nch > 1 && S < 5) return FP4_ERR_SHAPE;  // cannot happen (see launch_gemv); never run a partial K
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
    const int nt = (int)per;
    switch (S) {
    case 1: launch_gemv_nt<1>(g, nt, (unsigned)G, st); break;
    case 2: launch_gemv_nt<2>(g, nt, (unsigned)G, st); break;
    case 3: launch_gemv_nt<3>(g, nt, (unsigned)G, st); break;
    case 4: launch_gemv_nt<4>(g, nt, (unsigned)G, st); break;
    case 5: launch_gemv_nt<5>(g, nt, (unsigned)G, st); break;
    case 6: launch_gemv_nt<6>(g, nt, (unsigned)G, st); break;
    case 7: launch_gemv_nt<7>(g, nt, (unsigned)G, st); break;
    case 8: launch_gemv_nt<8>(g, nt, (unsigned)G, st); break;
    default: return FP4_ERR_SHAPE;
    }
    return hipGetLastError() == hipSuccess ? FP4_OK : FP4_ERR_HIP;
}

}  // namespace fp4k
