// internal.h -- declarations shared by the libfp4blk translation units (not
// part of the public C ABI; see include/fp4blk.h for that).
#pragma once

#include <stdint.h>

#include <atomic>

#include "fp4blk.h"

namespace fp4k {

struct FastDiv;

// Number of per-workgroup partial maxima the per-tensor amax pass writes; the
// per-tensor quantize workspace holds this many floats.
constexpr unsigned kAmaxPartials = 1024;

// Largest element count a flat (rows * cols) kernel indexes with 32-bit units
// of 8 elements.
constexpr int64_t kMaxFlatElems = (int64_t(1) << 31) * 8 - 8;

inline size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

fp4_status launch_nvfp4_quantize(const void *x, fp4_dtype xt, int64_t rows, int64_t cols,
                                 int64_t ldx, uint8_t *codes, uint8_t *scales, float *tscale,
                                 fp4_scale_mode mode, void *ws, int32_t *nonfinite,
                                 hipStream_t st);
fp4_status launch_nvfp4_dequantize(const uint8_t *codes, const uint8_t *scales, const float *tscale,
                                   fp4_scale_mode mode, int64_t rows, int64_t cols, void *y,
                                   fp4_dtype yt, int64_t ldy, hipStream_t st);
// load-only pass over bytes (a multiple of 16) at buf on grid x 512 threads (measure.hip)
fp4_status launch_read_ceiling(const void *buf, size_t bytes, int grid, uint32_t *sink, hipStream_t st);
fp4_status launch_mxfp4_quantize(const void *x, fp4_dtype xt, int64_t rows, int64_t cols,
                                 int64_t ldx, uint8_t *codes, uint8_t *scales, fp4_mx_rule rule,
                                 int32_t *nonfinite, hipStream_t st);
// the same quantizer writing the segment-major layout (cols % 128 == 0)
fp4_status launch_mxfp4_quantize_seg(const void *x, fp4_dtype xt, int64_t rows, int64_t cols,
                                     int64_t ldx, uint8_t *codes_p, uint8_t *scales_p, fp4_mx_rule rule,
                                     int32_t *nonfinite, hipStream_t st);
fp4_status launch_mxfp8_quantize(const void *x, fp4_dtype xt, int64_t rows, int64_t cols,
                                 int64_t ldx, uint8_t *codes, uint8_t *scales, fp4_mx_rule rule,
                                 int32_t *nonfinite, hipStream_t st);
fp4_status launch_mxfp4_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t rows,
                                   int64_t cols, void *y, fp4_dtype yt, int64_t ldy,
                                   hipStream_t st);

// NVFP4 GEMMs.  A is bf16 (a_codes == nullptr) or NVFP4 (a_codes/a_scales/a_tscale).
struct NvGemmArgs {
    const uint16_t *a;      // bf16 [M][lda] (W4A16)
    int64_t lda;
    const uint8_t *a_codes; // NVFP4 A (W4A4): codes [M][K/2], scales [M][K/16], tscale
    const uint8_t *a_scales;
    const float *a_tscale;
    int a_per_row;
    const uint8_t *w_codes;  // W [N][K/2]
    const uint8_t *w_scales; // W [N][K/16]
    const float *w_tscale;   // [1]
    int64_t M, N, K;
    void *c;
    int c_bf16;
    int64_t ldc;
    // grouped (MoE) form, groups > 0: M is the number of grouped rows (rows of C),
    // group e owns rows group_offs[e] .. group_offs[e + 1] - 1 and multiplies them by
    // weight e (w_codes / w_scales advance by one [N][K] weight per group, w_tscale
    // by one float); grouped row t reads A row row_index[t] (of a_rows rows), or row
    // t when row_index is null
    int groups;
    const int32_t *group_offs;
    const int32_t *row_index;
    int64_t a_rows;
    // W in the decode (segment-major) layout of w_rows rows, this launch's weight
    // rows starting at row w_row0 (ring kernel, not grouped)
    int w_seg;
    int64_t w_rows, w_row0;
};

fp4_status launch_nvfp4_gemm(const NvGemmArgs &g, hipStream_t st);
// W4A16 prefill on a weight in the decode layout (NVFP4, or MXFP4 when mx)
fp4_status launch_gemm_w4a16_seg(const NvGemmArgs &g, bool mx, hipStream_t st);
// NVFP4 W4A4 on a weight in the decode layout
fp4_status launch_gemm_w4a4_seg(const NvGemmArgs &g, hipStream_t st);
// grouped GEMM on the ring kernel: F = 0 NVFP4 W4A16, 1 NVFP4 W4A4, 2 MXFP4 W4A16
fp4_status launch_grouped_gemm(const NvGemmArgs &g, int fmt, hipStream_t st);

// compute units of the current device (cached per device; 256 if unknown)
int device_cu_count();

// Raises kernel `fn`'s dynamic LDS limit to `bytes` on the current device, once
// per device: `done` holds one bit per device id (0..63).  Two threads making the
// first call on a device at once may both set the attribute, which is harmless
// (the same value); the bit is published with release / acquire ordering.
inline bool set_max_lds_once(const void *fn, int bytes, std::atomic<uint64_t> &done)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
    const uint64_t bit = uint64_t(1) << dev;
    if (done.load(std::memory_order_acquire) & bit) return true;
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess) return false;
    done.fetch_or(bit, std::memory_order_release);
    return true;
}

// W4A16 decode GEMV over weights in the decode layout (gemv_nv.hip)
struct GemvArgs {
    const uint16_t *a;        // bf16 [M][lda]
    int64_t lda;
    const uint8_t *w_codes;   // [K/128][N][64]
    const uint8_t *w_scales;  // NVFP4 [K/128][N][8] E4M3; MXFP4 [K/128][N][4] E8M0
    const float *w_tscale;    // [1] (NVFP4; unused for MXFP4)
    int M, N, K;
    int mx;                   // weights are MXFP4
    int rows_per_wg;          // set by the launcher
    void *c;
    int c_bf16;
    int64_t ldc;
};

fp4_status launch_pack_decode(const uint8_t *codes, const uint8_t *scales, int64_t N, int64_t K,
                              uint8_t *codes_p, uint8_t *scales_p, bool mx, hipStream_t st);
fp4_status launch_gemv_decode(GemvArgs g, hipStream_t st);

// W4A16 prefill GEMM with MXFP4 weights (gemm_nv.hip; K % 128 == 0)
fp4_status launch_mxfp4_gemm_w4a16(const NvGemmArgs &g, hipStream_t st);

struct MxGemmArgs {
    const uint8_t *a_codes;  // [M][K/2]
    const uint8_t *a_scales; // [M][K/32]
    const uint8_t *w_codes;  // [N][K/2]
    const uint8_t *w_scales; // [N][K/32]
    int64_t M, N, K;
    void *c;
    int c_bf16;
    int64_t ldc;
    int w_seg;  // W4A8: W in the segment-major layout ([K/128][N][64], [K/128][N][4])
    // segment kernel: this launch's N columns are W rows w_row0 .. w_row0 + N - 1
    // of a weight of w_rows rows (0: the launch's N), so a launch can take the
    // last columns of a weight whose segment-major layout interleaves all rows
    int64_t w_row0, w_rows;
};

fp4_status launch_mxfp4_gemm(const MxGemmArgs &g, hipStream_t st);
// Both operands segment-major (codes [K/128][rows][64], scales [K/128][rows][4]);
// K % 128 == 0
fp4_status launch_mxfp4_gemm_seg(const MxGemmArgs &g, hipStream_t st);
// The same kernel with W row-major (A segment-major)
fp4_status launch_mxfp4_gemm_seg_wrow(const MxGemmArgs &g, hipStream_t st);
// W4A8: A MXFP8 (E4M3 bytes [M][K], E8M0 [M][K/32]), W MXFP4; K % 128 == 0
fp4_status launch_mxfp4_gemm_w4a8(const MxGemmArgs &g, hipStream_t st);

}  // namespace fp4k

// host-side construction of the device divider
#include "device_common.h"

namespace fp4k {
inline FastDiv make_fastdiv(uint32_t d)
{
    uint32_t s = 0;
    while ((uint64_t(1) << s) < d) ++s;
    const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << s) - d)) / d + 1;
    FastDiv f;
    f.d = d;
    f.m = (uint32_t)m;
    f.s = s;
    return f;
}
}  // namespace fp4k
