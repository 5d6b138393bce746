// abi.hip -- the extern "C" entry points of libfp4blk: argument validation,
// workspace layout and dispatch to the kernels.  Validation happens on the host
// before anything is launched, so an error leaves every output untouched.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "fp4blk.h"
#include "internal.h"

using namespace fp4k;

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

fp4_status check_device()
{
    int dev = 0;
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
        (void)hipGetLastError();
        return FP4_ERR_NO_DEVICE;
    }
    if (hipGetDevice(&dev) != hipSuccess) return FP4_ERR_NO_DEVICE;
    if (dev < 0 || dev >= kMaxDevices) return FP4_ERR_UNSUPPORTED_DEVICE;
    int st = g_dev_state[dev].load(std::memory_order_relaxed);
    if (st == 0) {
        hipDeviceProp_t p;
        if (hipGetDeviceProperties(&p, dev) != hipSuccess) return FP4_ERR_HIP;
        st = std::strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_dev_state[dev].store(st, std::memory_order_relaxed);
    }
    return st == 1 ? FP4_OK : FP4_ERR_UNSUPPORTED_DEVICE;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t dsize(fp4_dtype t) { return t == FP4_F32 ? 4 : 2; }

bool valid_dtype(int t) { return t == FP4_F32 || t == FP4_BF16; }

// Kernels that address an operand with 32-bit buffer offsets take operands under
// 2 GiB; the entry points check this on the host, before anything is launched.
constexpr int64_t k2GiB = int64_t(1) << 31;

// M rows and N rows of row_bytes each both stay under 2 GiB
bool codes_under_2gib(int64_t M, int64_t N, int64_t row_bytes)
{
    return M * row_bytes < k2GiB && N * row_bytes < k2GiB;
}

// rows x cols input with leading dimension ld (elements of size es): rows stay
// 16-byte aligned when the base is and ld * es is a multiple of 16.
fp4_status check_matrix(const void *p, int64_t rows, int64_t cols, int64_t ld, size_t es)
{
    if (!p) return FP4_ERR_NULL;
    if (rows <= 0 || cols <= 0) return FP4_ERR_SHAPE;
    if (ld < cols) return FP4_ERR_LAYOUT;
    if (!aligned16(p) || ((uint64_t)ld * es) % 16 != 0) return FP4_ERR_LAYOUT;
    return FP4_OK;
}

// packed operand (codes, scales): codes rows are cols/2 bytes, scale rows
// cols/block bytes; base pointers 16-byte aligned.
fp4_status check_packed(const uint8_t *codes, const uint8_t *scales)
{
    if (!codes || !scales) return FP4_ERR_NULL;
    if (!aligned16(codes) || !aligned16(scales)) return FP4_ERR_LAYOUT;
    return FP4_OK;
}

#define FP4_TRY(expr)                          \
    do {                                       \
        const fp4_status _s = (expr);          \
        if (_s != FP4_OK) return _s;           \
    } while (0)

}  // namespace

extern "C" {

const char *fp4_status_str(int s)
{
    switch (s) {
    case FP4_OK: return "FP4_OK";
    case FP4_ERR_NULL: return "FP4_ERR_NULL: a required pointer is null";
    case FP4_ERR_SHAPE: return "FP4_ERR_SHAPE: size <= 0, too large, or not a whole number of blocks";
    case FP4_ERR_LAYOUT: return "FP4_ERR_LAYOUT: leading dimension too small or pointer/row not 16-byte aligned";
    case FP4_ERR_DTYPE: return "FP4_ERR_DTYPE: unknown dtype, scale mode or MX rule";
    case FP4_ERR_WORKSPACE: return "FP4_ERR_WORKSPACE: workspace null or too small";
    case FP4_ERR_NO_DEVICE: return "FP4_ERR_NO_DEVICE: no HIP device visible";
    case FP4_ERR_UNSUPPORTED_DEVICE: return "FP4_ERR_UNSUPPORTED_DEVICE: current device is not gfx950";
    case FP4_ERR_HIP: return "FP4_ERR_HIP: a HIP call or kernel launch failed";
    default: return "unknown fp4_status";
    }
}

int fp4blk_version(void) { return 10000; }

fp4_status fp4blk_check_device(void) { return check_device(); }

fp4_status fp4blk_read_ceiling(const void *buf, size_t bytes, int grid, uint32_t *sink, hipStream_t stream)
{
    if (!buf || !sink) return FP4_ERR_NULL;
    if (bytes == 0 || bytes % 16 != 0 || grid <= 0 || grid > 65535) return FP4_ERR_SHAPE;
    if (!aligned16(buf)) return FP4_ERR_LAYOUT;
    FP4_TRY(check_device());
    return launch_read_ceiling(buf, bytes, grid, sink, stream);
}

// ------------------------------------------------------------------ NVFP4 --

size_t nvfp4_quantize_workspace(int64_t rows, int64_t cols, fp4_scale_mode mode)
{
    (void)rows;
    (void)cols;
    return mode == FP4_SCALE_PER_TENSOR ? kAmaxPartials * sizeof(float) : 0;
}

fp4_status nvfp4_quantize(const void *x, fp4_dtype xt, int64_t rows, int64_t cols, int64_t ldx,
                          uint8_t *codes, uint8_t *scales, float *tscale, fp4_scale_mode mode,
                          void *ws, size_t ws_bytes, int32_t *nonfinite, hipStream_t stream)
{
    if (!valid_dtype(xt) || (mode != FP4_SCALE_PER_TENSOR && mode != FP4_SCALE_PER_ROW))
        return FP4_ERR_DTYPE;
    FP4_TRY(check_matrix(x, rows, cols, ldx, dsize(xt)));
    if (cols % 16 != 0) return FP4_ERR_SHAPE;
    if (rows * cols > kMaxFlatElems) return FP4_ERR_SHAPE;
    if (!tscale) return FP4_ERR_NULL;
    FP4_TRY(check_packed(codes, scales));
    if (mode == FP4_SCALE_PER_TENSOR &&
        (!ws || ws_bytes < nvfp4_quantize_workspace(rows, cols, mode)))
        return FP4_ERR_WORKSPACE;
    FP4_TRY(check_device());
    return launch_nvfp4_quantize(x, xt, rows, cols, ldx, codes, scales, tscale, mode, ws, nonfinite,
                                 stream);
}

fp4_status nvfp4_dequantize(const uint8_t *codes, const uint8_t *scales, const float *tscale,
                            fp4_scale_mode mode, int64_t rows, int64_t cols, void *y,
                            fp4_dtype yt, int64_t ldy, hipStream_t stream)
{
    if (!valid_dtype(yt) || (mode != FP4_SCALE_PER_TENSOR && mode != FP4_SCALE_PER_ROW))
        return FP4_ERR_DTYPE;
    FP4_TRY(check_matrix(y, rows, cols, ldy, dsize(yt)));
    if (cols % 16 != 0) return FP4_ERR_SHAPE;
    if (rows * cols > kMaxFlatElems) return FP4_ERR_SHAPE;
    if (!tscale) return FP4_ERR_NULL;
    FP4_TRY(check_packed(codes, scales));
    FP4_TRY(check_device());
    return launch_nvfp4_dequantize(codes, scales, tscale, mode, rows, cols, y, yt, ldy, stream);
}

static fp4_status check_gemm_common(int64_t M, int64_t K, int64_t N, int kblock, const void *c,
                                    fp4_dtype ct, int64_t ldc)
{
    if (!valid_dtype(ct)) return FP4_ERR_DTYPE;
    if (M <= 0 || N <= 0 || K <= 0 || K % kblock != 0) return FP4_ERR_SHAPE;
    if (M > INT32_MAX / 2 || N > INT32_MAX / 2 || K > INT32_MAX / 2) return FP4_ERR_SHAPE;
    if (!c) return FP4_ERR_NULL;
    if (ldc < N) return FP4_ERR_LAYOUT;
    return FP4_OK;
}

fp4_status gemm_w4a16(const void *a, int64_t M, int64_t K, int64_t lda, const uint8_t *w_codes,
                      const uint8_t *w_scales, const float *w_tscale, int64_t N, void *c,
                      fp4_dtype ct, int64_t ldc, hipStream_t stream)
{
    FP4_TRY(check_gemm_common(M, K, N, 16, c, ct, ldc));
    FP4_TRY(check_matrix(a, M, K, lda, 2));
    FP4_TRY(check_packed(w_codes, w_scales));
    if (!w_tscale) return FP4_ERR_NULL;
    FP4_TRY(check_device());
    NvGemmArgs g{};
    g.a = reinterpret_cast<const uint16_t *>(a);
    g.lda = lda;
    g.w_codes = w_codes;
    g.w_scales = w_scales;
    g.w_tscale = w_tscale;
    g.M = M;
    g.N = N;
    g.K = K;
    g.c = c;
    g.c_bf16 = ct == FP4_BF16;
    g.ldc = ldc;
    return launch_nvfp4_gemm(g, stream);
}

fp4_status nvfp4_pack_decode(const uint8_t *codes, const uint8_t *scales, int64_t N, int64_t K,
                             uint8_t *codes_p, uint8_t *scales_p, hipStream_t stream)
{
    if (N <= 0 || K <= 0 || K % 128 != 0 || N > INT32_MAX / 2 || K > INT32_MAX / 2) return FP4_ERR_SHAPE;
    FP4_TRY(check_packed(codes, scales));
    FP4_TRY(check_packed(codes_p, scales_p));
    FP4_TRY(check_device());
    return launch_pack_decode(codes, scales, N, K, codes_p, scales_p, false, stream);
}

namespace {

// Both kernels behind the decode-layout entry points address A and the weight
// with 32-bit byte offsets (the GEMV's buffer descriptors hold 32-bit sizes, and
// its out-of-range offset 2^31 must lie past every operand): A's bytes up to its
// last element and the weight's code bytes stay below 2^31 for every M.
fp4_status check_decode_limits(int64_t M, int64_t K, int64_t lda, int64_t N)
{
    if ((M - 1) * lda * 2 + K * 2 >= k2GiB || M * lda * 2 >= k2GiB) return FP4_ERR_SHAPE;
    if (N * (K / 2) >= k2GiB) return FP4_ERR_SHAPE;
    return FP4_OK;
}

// M > 16 on a decode-layout weight: the prefill ring kernel reading that layout
fp4_status w4a16_seg_prefill(const void *a, int64_t M, int64_t K, int64_t lda, const uint8_t *w_codes_p,
                             const uint8_t *w_scales_p, const float *w_tscale, int64_t N, void *c, fp4_dtype ct,
                             int64_t ldc, bool mx, hipStream_t stream)
{
    NvGemmArgs g{};
    g.a = reinterpret_cast<const uint16_t *>(a);
    g.lda = lda;
    g.w_codes = w_codes_p;
    g.w_scales = w_scales_p;
    g.w_tscale = w_tscale;
    g.M = M;
    g.N = N;
    g.K = K;
    g.c = c;
    g.c_bf16 = ct == FP4_BF16;
    g.ldc = ldc;
    g.w_seg = 1;
    g.w_rows = N;
    g.w_row0 = 0;
    return launch_gemm_w4a16_seg(g, mx, stream);
}

}  // namespace

fp4_status gemm_w4a16_decode(const void *a, int64_t M, int64_t K, int64_t lda, const uint8_t *w_codes_p,
                             const uint8_t *w_scales_p, const float *w_tscale, int64_t N, void *c,
                             fp4_dtype ct, int64_t ldc, hipStream_t stream)
{
    FP4_TRY(check_gemm_common(M, K, N, 128, c, ct, ldc));
    FP4_TRY(check_matrix(a, M, K, lda, 2));
    FP4_TRY(check_decode_limits(M, K, lda, N));
    FP4_TRY(check_packed(w_codes_p, w_scales_p));
    if (!w_tscale) return FP4_ERR_NULL;
    FP4_TRY(check_device());
    if (M > 16) return w4a16_seg_prefill(a, M, K, lda, w_codes_p, w_scales_p, w_tscale, N, c, ct, ldc, false, stream);
    GemvArgs g{};
    g.a = reinterpret_cast<const uint16_t *>(a);
    g.lda = lda;
    g.w_codes = w_codes_p;
    g.w_scales = w_scales_p;
    g.w_tscale = w_tscale;
    g.M = (int)M;
    g.N = (int)N;
    g.K = (int)K;
    g.c = c;
    g.c_bf16 = ct == FP4_BF16;
    g.ldc = ldc;
    return launch_gemv_decode(g, stream);
}

fp4_status mxfp4_pack_decode(const uint8_t *codes, const uint8_t *scales, int64_t N, int64_t K,
                             uint8_t *codes_p, uint8_t *scales_p, hipStream_t stream)
{
    if (N <= 0 || K <= 0 || K % 128 != 0 || N > INT32_MAX / 2 || K > INT32_MAX / 2) return FP4_ERR_SHAPE;
    FP4_TRY(check_packed(codes, scales));
    FP4_TRY(check_packed(codes_p, scales_p));
    FP4_TRY(check_device());
    return launch_pack_decode(codes, scales, N, K, codes_p, scales_p, true, stream);
}

fp4_status mxfp4_gemm_w4a16_decode(const void *a, int64_t M, int64_t K, int64_t lda, const uint8_t *w_codes_p,
                                   const uint8_t *w_scales_p, int64_t N, void *c, fp4_dtype ct, int64_t ldc,
                                   hipStream_t stream)
{
    FP4_TRY(check_gemm_common(M, K, N, 128, c, ct, ldc));
    FP4_TRY(check_matrix(a, M, K, lda, 2));
    FP4_TRY(check_decode_limits(M, K, lda, N));
    FP4_TRY(check_packed(w_codes_p, w_scales_p));
    FP4_TRY(check_device());
    if (M > 16) return w4a16_seg_prefill(a, M, K, lda, w_codes_p, w_scales_p, nullptr, N, c, ct, ldc, true, stream);
    GemvArgs g{};
    g.a = reinterpret_cast<const uint16_t *>(a);
    g.lda = lda;
    g.w_codes = w_codes_p;
    g.w_scales = w_scales_p;
    g.w_tscale = nullptr;
    g.M = (int)M;
    g.N = (int)N;
    g.K = (int)K;
    g.mx = 1;
    g.c = c;
    g.c_bf16 = ct == FP4_BF16;
    g.ldc = ldc;
    return launch_gemv_decode(g, stream);
}

fp4_status mxfp4_gemm_w4a16(const void *a, int64_t M, int64_t K, int64_t lda, const uint8_t *w_codes,
                            const uint8_t *w_scales, int64_t N, void *c, fp4_dtype ct, int64_t ldc,
                            hipStream_t stream)
{
    FP4_TRY(check_gemm_common(M, K, N, 128, c, ct, ldc));
    FP4_TRY(check_matrix(a, M, K, lda, 2));
    FP4_TRY(check_packed(w_codes, w_scales));
    FP4_TRY(check_device());
    NvGemmArgs g{};
    g.a = reinterpret_cast<const uint16_t *>(a);
    g.lda = lda;
    g.w_codes = w_codes;
    g.w_scales = w_scales;
    g.w_tscale = nullptr;
    g.M = M;
    g.N = N;
    g.K = K;
    g.c = c;
    g.c_bf16 = ct == FP4_BF16;
    g.ldc = ldc;
    return launch_mxfp4_gemm_w4a16(g, stream);
}

void gemm_w4a4_workspace_offsets(int64_t M, int64_t K, size_t *codes_off, size_t *scales_off,
                                 size_t *tscale_off)
{
    const size_t cb = align256((size_t)M * (size_t)(K / 2));
    const size_t sb = align256((size_t)M * (size_t)(K / 16));
    if (codes_off) *codes_off = 0;
    if (scales_off) *scales_off = cb;
    if (tscale_off) *tscale_off = cb + sb;
}

size_t gemm_w4a4_workspace(int64_t M, int64_t K, fp4_scale_mode a_mode)
{
    if (M <= 0 || K <= 0) return 0;
    size_t t;
    gemm_w4a4_workspace_offsets(M, K, nullptr, nullptr, &t);
    const size_t ts = align256((size_t)(a_mode == FP4_SCALE_PER_ROW ? M : 1) * sizeof(float));
    // the per-tensor amax partials follow the tensor scale
    const size_t amax = a_mode == FP4_SCALE_PER_TENSOR ? kAmaxPartials * sizeof(float) : 0;
    return t + ts + amax;
}

namespace {

// the GEMM half of the NVFP4 W4A4 forms, arguments checked (w_seg: W in the decode layout)
fp4_status w4a4_launch(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_tscale, fp4_scale_mode a_mode,
                       int64_t M, int64_t K, const uint8_t *w_codes, const uint8_t *w_scales, const float *w_tscale,
                       int64_t N, void *c, fp4_dtype ct, int64_t ldc, bool w_seg, hipStream_t stream)
{
    NvGemmArgs g{};
    g.a_codes = a_codes;
    g.a_scales = a_scales;
    g.a_tscale = a_tscale;
    g.a_per_row = a_mode == FP4_SCALE_PER_ROW;
    g.w_codes = w_codes;
    g.w_scales = w_scales;
    g.w_tscale = w_tscale;
    g.M = M;
    g.N = N;
    g.K = K;
    g.c = c;
    g.c_bf16 = ct == FP4_BF16;
    g.ldc = ldc;
    if (!w_seg) return launch_nvfp4_gemm(g, stream);
    g.w_seg = 1;
    g.w_rows = N;
    g.w_row0 = 0;
    return launch_gemm_w4a4_seg(g, stream);
}

fp4_status w4a4_prequant(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_tscale, fp4_scale_mode a_mode,
                         int64_t M, int64_t K, const uint8_t *w_codes, const uint8_t *w_scales, const float *w_tscale,
                         int64_t N, void *c, fp4_dtype ct, int64_t ldc, bool w_seg, hipStream_t stream)
{
    if (a_mode != FP4_SCALE_PER_TENSOR && a_mode != FP4_SCALE_PER_ROW) return FP4_ERR_DTYPE;
    FP4_TRY(check_gemm_common(M, K, N, w_seg ? 128 : 16, c, ct, ldc));
    FP4_TRY(check_packed(a_codes, a_scales));
    FP4_TRY(check_packed(w_codes, w_scales));
    if (!a_tscale || !w_tscale) return FP4_ERR_NULL;
    if (w_seg && !codes_under_2gib(M, N, K / 2)) return FP4_ERR_SHAPE;
    FP4_TRY(check_device());
    return w4a4_launch(a_codes, a_scales, a_tscale, a_mode, M, K, w_codes, w_scales, w_tscale, N, c, ct, ldc, w_seg,
                       stream);
}

fp4_status w4a4_full(const void *a, int64_t M, int64_t K, int64_t lda, fp4_scale_mode a_mode, const uint8_t *w_codes,
                     const uint8_t *w_scales, const float *w_tscale, int64_t N, void *c, fp4_dtype ct, int64_t ldc,
                     void *ws, size_t ws_bytes, bool w_seg, hipStream_t stream)
{
    if (a_mode != FP4_SCALE_PER_TENSOR && a_mode != FP4_SCALE_PER_ROW) return FP4_ERR_DTYPE;
    FP4_TRY(check_gemm_common(M, K, N, w_seg ? 128 : 16, c, ct, ldc));
    FP4_TRY(check_matrix(a, M, K, lda, 2));
    if (M * K > kMaxFlatElems) return FP4_ERR_SHAPE;
    FP4_TRY(check_packed(w_codes, w_scales));
    if (!w_tscale) return FP4_ERR_NULL;
    if (!ws || !aligned16(ws) || ws_bytes < gemm_w4a4_workspace(M, K, a_mode))
        return FP4_ERR_WORKSPACE;
    if (w_seg && !codes_under_2gib(M, N, K / 2)) return FP4_ERR_SHAPE;  // before A is quantized
    FP4_TRY(check_device());
    size_t co, so, to;
    gemm_w4a4_workspace_offsets(M, K, &co, &so, &to);
    uint8_t *base = reinterpret_cast<uint8_t *>(ws);
    uint8_t *ac = base + co;
    uint8_t *as = base + so;
    float *at = reinterpret_cast<float *>(base + to);
    void *amax_ws = base + to + align256((size_t)(a_mode == FP4_SCALE_PER_ROW ? M : 1) * sizeof(float));
    FP4_TRY(launch_nvfp4_quantize(a, FP4_BF16, M, K, lda, ac, as, at, a_mode, amax_ws, nullptr,
                                  stream));
    return w4a4_launch(ac, as, at, a_mode, M, K, w_codes, w_scales, w_tscale, N, c, ct, ldc, w_seg, stream);
}

}  // namespace

fp4_status gemm_nvfp4_w4a4_prequant(const uint8_t *a_codes, const uint8_t *a_scales,
                                    const float *a_tscale, fp4_scale_mode a_mode, int64_t M,
                                    int64_t K, const uint8_t *w_codes, const uint8_t *w_scales,
                                    const float *w_tscale, int64_t N, void *c, fp4_dtype ct,
                                    int64_t ldc, hipStream_t stream)
{
    return w4a4_prequant(a_codes, a_scales, a_tscale, a_mode, M, K, w_codes, w_scales, w_tscale, N, c, ct, ldc, false,
                         stream);
}

fp4_status gemm_w4a4(const void *a, int64_t M, int64_t K, int64_t lda, fp4_scale_mode a_mode,
                     const uint8_t *w_codes, const uint8_t *w_scales, const float *w_tscale,
                     int64_t N, void *c, fp4_dtype ct, int64_t ldc, void *ws, size_t ws_bytes,
                     hipStream_t stream)
{
    return w4a4_full(a, M, K, lda, a_mode, w_codes, w_scales, w_tscale, N, c, ct, ldc, ws, ws_bytes, false, stream);
}

fp4_status gemm_nvfp4_w4a4_prequant_seg(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_tscale,
                                        fp4_scale_mode a_mode, int64_t M, int64_t K, const uint8_t *w_codes_p,
                                        const uint8_t *w_scales_p, const float *w_tscale, int64_t N, void *c,
                                        fp4_dtype ct, int64_t ldc, hipStream_t stream)
{
    return w4a4_prequant(a_codes, a_scales, a_tscale, a_mode, M, K, w_codes_p, w_scales_p, w_tscale, N, c, ct, ldc,
                         true, stream);
}

fp4_status gemm_w4a4_seg(const void *a, int64_t M, int64_t K, int64_t lda, fp4_scale_mode a_mode,
                         const uint8_t *w_codes_p, const uint8_t *w_scales_p, const float *w_tscale, int64_t N,
                         void *c, fp4_dtype ct, int64_t ldc, void *ws, size_t ws_bytes, hipStream_t stream)
{
    return w4a4_full(a, M, K, lda, a_mode, w_codes_p, w_scales_p, w_tscale, N, c, ct, ldc, ws, ws_bytes, true, stream);
}

}  // extern "C"

// ------------------------------------------------ W4A4 without allocation --
//
// gemm_w4a4_noalloc keeps A's packed form in `scratch`, a device array of the
// library itself, instead of a caller's workspace.  Each device holds its own
// copy from the time the library's code is loaded on it until the process ends.
// In host code `scratch` names a host-side stand-in, never device memory: its
// device address is looked up once per device (hipGetSymbolAddress, with that
// device current) and only that address is passed to kernels.  Nothing in it
// needs clearing between calls: the quantizer writes every byte the GEMM reads
// (codes, scales, tensor scales and, per tensor, all amax partials it reduces).

namespace {

constexpr size_t kNoallocScratchBytes = size_t(32) << 20;

static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

std::atomic<uintptr_t> g_scratch_addr[kMaxDevices];  // 0 until looked up on that device

// The device address of the current device's `scratch`, or null on failure.
void *scratch_on_current_device()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    uintptr_t p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        void *q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) {
            (void)hipGetLastError();
            return nullptr;
        }
        p = reinterpret_cast<uintptr_t>(q);
        g_scratch_addr[dev].store(p, std::memory_order_release);  // racing first calls store the same address
    }
    return reinterpret_cast<void *>(p);
}

}  // namespace

extern "C" {

fp4_status gemm_w4a4_noalloc(const void *a, int64_t M, int64_t K, int64_t lda, fp4_scale_mode a_mode,
                             const uint8_t *w_codes, const uint8_t *w_scales, const float *w_tscale, int64_t N,
                             void *c, fp4_dtype ct, int64_t ldc, hipStream_t stream)
{
    if (a_mode != FP4_SCALE_PER_TENSOR && a_mode != FP4_SCALE_PER_ROW) return FP4_ERR_DTYPE;
    FP4_TRY(check_gemm_common(M, K, N, 16, c, ct, ldc));
    FP4_TRY(check_matrix(a, M, K, lda, 2));
    if (M * K > kMaxFlatElems) return FP4_ERR_SHAPE;
    FP4_TRY(check_packed(w_codes, w_scales));
    if (!w_tscale) return FP4_ERR_NULL;
    if (gemm_w4a4_workspace(M, K, a_mode) > kNoallocScratchBytes) return FP4_ERR_WORKSPACE;
    FP4_TRY(check_device());
    void *ws = scratch_on_current_device();
    if (!ws) return FP4_ERR_HIP;
    return w4a4_full(a, M, K, lda, a_mode, w_codes, w_scales, w_tscale, N, c, ct, ldc, ws, kNoallocScratchBytes, false,
                     stream);
}

// ------------------------------------------------------------------ MXFP4 --

fp4_status mxfp4_quantize(const void *x, fp4_dtype xt, int64_t rows, int64_t cols, int64_t ldx,
                          uint8_t *codes, uint8_t *scales, fp4_mx_rule rule, int32_t *nonfinite,
                          hipStream_t stream)
{
    if (!valid_dtype(xt) || (rule != FP4_MX_OCP_FLOOR && rule != FP4_MX_CEIL)) return FP4_ERR_DTYPE;
    FP4_TRY(check_matrix(x, rows, cols, ldx, dsize(xt)));
    if (cols % 32 != 0) return FP4_ERR_SHAPE;
    if (rows * cols > kMaxFlatElems) return FP4_ERR_SHAPE;
    FP4_TRY(check_packed(codes, scales));
    FP4_TRY(check_device());
    return launch_mxfp4_quantize(x, xt, rows, cols, ldx, codes, scales, rule, nonfinite, stream);
}

fp4_status mxfp4_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t rows,
                            int64_t cols, void *y, fp4_dtype yt, int64_t ldy, hipStream_t stream)
{
    if (!valid_dtype(yt)) return FP4_ERR_DTYPE;
    FP4_TRY(check_matrix(y, rows, cols, ldy, dsize(yt)));
    if (cols % 32 != 0) return FP4_ERR_SHAPE;
    if (rows * cols > kMaxFlatElems) return FP4_ERR_SHAPE;
    FP4_TRY(check_packed(codes, scales));
    FP4_TRY(check_device());
    return launch_mxfp4_dequantize(codes, scales, rows, cols, y, yt, ldy, stream);
}

size_t mxfp4_gemm_w4a4_workspace(int64_t M, int64_t K)
{
    if (M <= 0 || K <= 0) return 0;
    return align256((size_t)M * (size_t)(K / 2)) + align256((size_t)M * (size_t)(K / 32));
}

fp4_status mxfp4_gemm_prequant(const uint8_t *a_codes, const uint8_t *a_scales, int64_t M,
                               int64_t K, const uint8_t *w_codes, const uint8_t *w_scales,
                               int64_t N, void *c, fp4_dtype ct, int64_t ldc, hipStream_t stream)
{
    FP4_TRY(check_gemm_common(M, K, N, 32, c, ct, ldc));
    FP4_TRY(check_packed(a_codes, a_scales));
    FP4_TRY(check_packed(w_codes, w_scales));
    FP4_TRY(check_device());
    MxGemmArgs g{};
    g.a_codes = a_codes;
    g.a_scales = a_scales;
    g.w_codes = w_codes;
    g.w_scales = w_scales;
    g.M = M;
    g.N = N;
    g.K = K;
    g.c = c;
    g.c_bf16 = ct == FP4_BF16;
    g.ldc = ldc;
    return launch_mxfp4_gemm(g, stream);
}

int mxfp4_gemm_w4a4_a_segment_major(int64_t M, int64_t N, int64_t K)
{
    return M > 0 && N > 0 && K > 0 && K % 128 == 0 && codes_under_2gib(M, N, K / 2) ? 1 : 0;
}

fp4_status mxfp4_gemm_w4a4(const void *a, int64_t M, int64_t K, int64_t lda, fp4_mx_rule rule,
                           const uint8_t *w_codes, const uint8_t *w_scales, int64_t N, void *c,
                           fp4_dtype ct, int64_t ldc, void *ws, size_t ws_bytes,
                           hipStream_t stream)
{
    if (rule != FP4_MX_OCP_FLOOR && rule != FP4_MX_CEIL) return FP4_ERR_DTYPE;
    FP4_TRY(check_gemm_common(M, K, N, 32, c, ct, ldc));
    FP4_TRY(check_matrix(a, M, K, lda, 2));
    if (M * K > kMaxFlatElems) return FP4_ERR_SHAPE;
    FP4_TRY(check_packed(w_codes, w_scales));
    if (!ws || !aligned16(ws) || ws_bytes < mxfp4_gemm_w4a4_workspace(M, K)) return FP4_ERR_WORKSPACE;
    FP4_TRY(check_device());
    uint8_t *ac = reinterpret_cast<uint8_t *>(ws);
    uint8_t *as = ac + align256((size_t)M * (size_t)(K / 2));
    // A's packed form lives only in the workspace, so its layout is this call's
    // choice: segment-major (each 256-row panel's 128-K segment one contiguous
    // 16 KiB run) whenever the segment kernel applies, with W read row-major by
    // the same kernel; the products and their order, and so C, are the same
    const bool seg = mxfp4_gemm_w4a4_a_segment_major(M, N, K) != 0;
    if (seg)
        FP4_TRY(launch_mxfp4_quantize_seg(a, FP4_BF16, M, K, lda, ac, as, rule, nullptr, stream));
    else
        FP4_TRY(launch_mxfp4_quantize(a, FP4_BF16, M, K, lda, ac, as, rule, nullptr, stream));
    MxGemmArgs g{};
    g.a_codes = ac;
    g.a_scales = as;
    g.w_codes = w_codes;
    g.w_scales = w_scales;
    g.M = M;
    g.N = N;
    g.K = K;
    g.c = c;
    g.c_bf16 = ct == FP4_BF16;
    g.ldc = ldc;
    return seg ? launch_mxfp4_gemm_seg_wrow(g, stream) : launch_mxfp4_gemm(g, stream);
}

// ------------------------------------------- MXFP4 W4A4, segment-major ----

size_t mxfp4_gemm_w4a4_seg_workspace(int64_t M, int64_t K)
{
    return mxfp4_gemm_w4a4_workspace(M, K);  // the same bytes, in the other order
}

fp4_status mxfp4_gemm_prequant_seg(const uint8_t *a_codes_p, const uint8_t *a_scales_p, int64_t M, int64_t K,
                                   const uint8_t *w_codes_p, const uint8_t *w_scales_p, int64_t N, void *c,
                                   fp4_dtype ct, int64_t ldc, hipStream_t stream)
{
    FP4_TRY(check_gemm_common(M, K, N, 128, c, ct, ldc));
    FP4_TRY(check_packed(a_codes_p, a_scales_p));
    FP4_TRY(check_packed(w_codes_p, w_scales_p));
    if (!codes_under_2gib(M, N, K / 2)) return FP4_ERR_SHAPE;
    FP4_TRY(check_device());
    MxGemmArgs g{};
    g.a_codes = a_codes_p;
    g.a_scales = a_scales_p;
    g.w_codes = w_codes_p;
    g.w_scales = w_scales_p;
    g.M = M;
    g.N = N;
    g.K = K;
    g.c = c;
    g.c_bf16 = ct == FP4_BF16;
    g.ldc = ldc;
    return launch_mxfp4_gemm_seg(g, stream);
}

fp4_status mxfp4_gemm_w4a4_seg(const void *a, int64_t M, int64_t K, int64_t lda, fp4_mx_rule rule,
                               const uint8_t *w_codes_p, const uint8_t *w_scales_p, int64_t N, void *c,
                               fp4_dtype ct, int64_t ldc, void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (rule != FP4_MX_OCP_FLOOR && rule != FP4_MX_CEIL) return FP4_ERR_DTYPE;
    FP4_TRY(check_gemm_common(M, K, N, 128, c, ct, ldc));
    FP4_TRY(check_matrix(a, M, K, lda, 2));
    if (M * K > kMaxFlatElems) return FP4_ERR_SHAPE;
    FP4_TRY(check_packed(w_codes_p, w_scales_p));
    if (!ws || !aligned16(ws) || ws_bytes < mxfp4_gemm_w4a4_seg_workspace(M, K)) return FP4_ERR_WORKSPACE;
    if (!codes_under_2gib(M, N, K / 2)) return FP4_ERR_SHAPE;  // before A is quantized
    FP4_TRY(check_device());
    uint8_t *ac = reinterpret_cast<uint8_t *>(ws);
    uint8_t *as = ac + align256((size_t)M * (size_t)(K / 2));
    FP4_TRY(launch_mxfp4_quantize_seg(a, FP4_BF16, M, K, lda, ac, as, rule, nullptr, stream));
    MxGemmArgs g{};
    g.a_codes = ac;
    g.a_scales = as;
    g.w_codes = w_codes_p;
    g.w_scales = w_scales_p;
    g.M = M;
    g.N = N;
    g.K = K;
    g.c = c;
    g.c_bf16 = ct == FP4_BF16;
    g.ldc = ldc;
    return launch_mxfp4_gemm_seg(g, stream);
}

// ------------------------------------------------------------------- W4A8 --

fp4_status mxfp8_quantize(const void *x, fp4_dtype xt, int64_t rows, int64_t cols, int64_t ldx,
                          uint8_t *codes, uint8_t *scales, fp4_mx_rule rule, int32_t *nonfinite,
                          hipStream_t stream)
{
    if (!valid_dtype(xt) || (rule != FP4_MX_OCP_FLOOR && rule != FP4_MX_CEIL)) return FP4_ERR_DTYPE;
    FP4_TRY(check_matrix(x, rows, cols, ldx, dsize(xt)));
    if (cols % 32 != 0) return FP4_ERR_SHAPE;
    if (rows * cols > kMaxFlatElems) return FP4_ERR_SHAPE;
    FP4_TRY(check_packed(codes, scales));
    FP4_TRY(check_device());
    return launch_mxfp8_quantize(x, xt, rows, cols, ldx, codes, scales, rule, nonfinite, stream);
}

size_t mxfp4_gemm_w4a8_workspace(int64_t M, int64_t K)
{
    if (M <= 0 || K <= 0) return 0;
    return align256((size_t)M * (size_t)K) + align256((size_t)M * (size_t)(K / 32));
}

namespace {

// the GEMM half of both W4A8 forms (w_seg: W segment-major)
fp4_status w4a8_gemm(const uint8_t *a_codes, const uint8_t *a_scales, int64_t M, int64_t K, const uint8_t *w_codes,
                     const uint8_t *w_scales, int64_t N, void *c, fp4_dtype ct, int64_t ldc, bool w_seg,
                     hipStream_t stream)
{
    FP4_TRY(check_gemm_common(M, K, N, 128, c, ct, ldc));
    FP4_TRY(check_packed(a_codes, a_scales));
    FP4_TRY(check_packed(w_codes, w_scales));
    if (M * K >= k2GiB || !codes_under_2gib(0, N, K / 2)) return FP4_ERR_SHAPE;
    FP4_TRY(check_device());
    MxGemmArgs g{};
    g.a_codes = a_codes;
    g.a_scales = a_scales;
    g.w_codes = w_codes;
    g.w_scales = w_scales;
    g.M = M;
    g.N = N;
    g.K = K;
    g.c = c;
    g.c_bf16 = ct == FP4_BF16;
    g.ldc = ldc;
    g.w_seg = w_seg ? 1 : 0;
    return launch_mxfp4_gemm_w4a8(g, stream);
}

fp4_status w4a8_full(const void *a, int64_t M, int64_t K, int64_t lda, fp4_mx_rule rule, const uint8_t *w_codes,
                     const uint8_t *w_scales, int64_t N, void *c, fp4_dtype ct, int64_t ldc, void *ws,
                     size_t ws_bytes, bool w_seg, hipStream_t stream)
{
    if (rule != FP4_MX_OCP_FLOOR && rule != FP4_MX_CEIL) return FP4_ERR_DTYPE;
    FP4_TRY(check_gemm_common(M, K, N, 128, c, ct, ldc));
    FP4_TRY(check_matrix(a, M, K, lda, 2));
    if (M * K > kMaxFlatElems) return FP4_ERR_SHAPE;
    FP4_TRY(check_packed(w_codes, w_scales));
    if (!ws || !aligned16(ws) || ws_bytes < mxfp4_gemm_w4a8_workspace(M, K)) return FP4_ERR_WORKSPACE;
    if (M * K >= k2GiB || !codes_under_2gib(0, N, K / 2)) return FP4_ERR_SHAPE;  // before A is quantized
    FP4_TRY(check_device());
    uint8_t *ac = reinterpret_cast<uint8_t *>(ws);
    uint8_t *as = ac + align256((size_t)M * (size_t)K);
    FP4_TRY(launch_mxfp8_quantize(a, FP4_BF16, M, K, lda, ac, as, rule, nullptr, stream));
    return w4a8_gemm(ac, as, M, K, w_codes, w_scales, N, c, ct, ldc, w_seg, stream);
}

}  // namespace

fp4_status mxfp4_gemm_w4a8_prequant(const uint8_t *a_codes, const uint8_t *a_scales, int64_t M, int64_t K,
                                    const uint8_t *w_codes, const uint8_t *w_scales, int64_t N, void *c,
                                    fp4_dtype ct, int64_t ldc, hipStream_t stream)
{
    return w4a8_gemm(a_codes, a_scales, M, K, w_codes, w_scales, N, c, ct, ldc, false, stream);
}

fp4_status mxfp4_gemm_w4a8(const void *a, int64_t M, int64_t K, int64_t lda, fp4_mx_rule rule,
                           const uint8_t *w_codes, const uint8_t *w_scales, int64_t N, void *c,
                           fp4_dtype ct, int64_t ldc, void *ws, size_t ws_bytes, hipStream_t stream)
{
    return w4a8_full(a, M, K, lda, rule, w_codes, w_scales, N, c, ct, ldc, ws, ws_bytes, false, stream);
}

fp4_status mxfp4_gemm_w4a8_prequant_seg(const uint8_t *a_codes, const uint8_t *a_scales, int64_t M, int64_t K,
                                        const uint8_t *w_codes_p, const uint8_t *w_scales_p, int64_t N, void *c,
                                        fp4_dtype ct, int64_t ldc, hipStream_t stream)
{
    return w4a8_gemm(a_codes, a_scales, M, K, w_codes_p, w_scales_p, N, c, ct, ldc, true, stream);
}

fp4_status mxfp4_gemm_w4a8_seg(const void *a, int64_t M, int64_t K, int64_t lda, fp4_mx_rule rule,
                               const uint8_t *w_codes_p, const uint8_t *w_scales_p, int64_t N, void *c,
                               fp4_dtype ct, int64_t ldc, void *ws, size_t ws_bytes, hipStream_t stream)
{
    return w4a8_full(a, M, K, lda, rule, w_codes_p, w_scales_p, N, c, ct, ldc, ws, ws_bytes, true, stream);
}

// ------------------------------------------------------- grouped (MoE) --

namespace {

constexpr int64_t kMaxGroups = 1 << 16;

// Arguments every grouped GEMM shares.  rows == 0 (no routed rows) is valid: once
// the sizes and group arguments check out, *empty is set and the caller returns
// FP4_OK without touching A, W or C (which may then be empty, even null).
fp4_status check_grouped(int64_t a_rows, int64_t K, const int32_t *row_index, const int32_t *group_offs,
                         int64_t groups, int64_t rows, int64_t N, int kblock, const void *c, fp4_dtype ct,
                         int64_t ldc, bool *empty)
{
    if (rows < 0) return FP4_ERR_SHAPE;
    if (groups <= 0 || groups > kMaxGroups) return FP4_ERR_SHAPE;
    if (!group_offs) return FP4_ERR_NULL;
    *empty = rows == 0;
    if (*empty) {
        if (!valid_dtype(ct)) return FP4_ERR_DTYPE;
        return N > 0 && K > 0 && K % kblock == 0 ? FP4_OK : FP4_ERR_SHAPE;
    }
    FP4_TRY(check_gemm_common(rows, K, N, kblock, c, ct, ldc));
    if (a_rows <= 0 || a_rows > INT32_MAX / 2) return FP4_ERR_SHAPE;
    if (!row_index && a_rows < rows) return FP4_ERR_SHAPE;
    return FP4_OK;
}

// The grouped kernel's own limits, checked here so that nothing (not even the
// W4A4 activation quantizer) is launched for a call the kernel would refuse:
// 32-bit byte offsets into A (its bf16 rows, or its packed codes for W4A4) and
// into one group's weight codes, and a grid below 2^31 workgroups.
fp4_status check_grouped_limits(int64_t a_rows, int64_t K, int64_t lda, bool a_fp4, int64_t groups,
                                int64_t rows, int64_t N)
{
    const int64_t a_bytes = a_fp4 ? a_rows * (K / 2) : a_rows * lda * 2;
    if (a_bytes >= k2GiB || N * (K / 2) >= k2GiB) return FP4_ERR_SHAPE;
    if (((rows + 127) / 128 + groups) * ((N + 255) / 256) >= k2GiB) return FP4_ERR_SHAPE;
    return FP4_OK;
}

NvGemmArgs grouped_args(int64_t a_rows, int64_t K, const int32_t *row_index, const int32_t *group_offs,
                        int64_t groups, int64_t rows, const uint8_t *w_codes, const uint8_t *w_scales,
                        const float *w_tscale, int64_t N, void *c, fp4_dtype ct, int64_t ldc)
{
    NvGemmArgs g{};
    g.w_codes = w_codes;
    g.w_scales = w_scales;
    g.w_tscale = w_tscale;
    g.M = rows;
    g.N = N;
    g.K = K;
    g.c = c;
    g.c_bf16 = ct == FP4_BF16;
    g.ldc = ldc;
    g.groups = (int)groups;
    g.group_offs = group_offs;
    g.row_index = row_index;
    g.a_rows = a_rows;
    return g;
}

}  // namespace

fp4_status nvfp4_grouped_gemm_w4a16(const void *a, int64_t a_rows, int64_t K, int64_t lda,
                                    const int32_t *row_index, const int32_t *group_offs, int64_t groups,
                                    int64_t rows, const uint8_t *w_codes, const uint8_t *w_scales,
                                    const float *w_tscale, int64_t N, void *c, fp4_dtype ct, int64_t ldc,
                                    hipStream_t stream)
{
    bool empty = false;
    FP4_TRY(check_grouped(a_rows, K, row_index, group_offs, groups, rows, N, 64, c, ct, ldc, &empty));
    if (empty) return FP4_OK;
    FP4_TRY(check_matrix(a, a_rows, K, lda, 2));
    FP4_TRY(check_grouped_limits(a_rows, K, lda, false, groups, rows, N));
    FP4_TRY(check_packed(w_codes, w_scales));
    if (!w_tscale) return FP4_ERR_NULL;
    FP4_TRY(check_device());
    NvGemmArgs g = grouped_args(a_rows, K, row_index, group_offs, groups, rows, w_codes, w_scales, w_tscale, N, c,
                                ct, ldc);
    g.a = reinterpret_cast<const uint16_t *>(a);
    g.lda = lda;
    return launch_grouped_gemm(g, 0, stream);
}

fp4_status mxfp4_grouped_gemm_w4a16(const void *a, int64_t a_rows, int64_t K, int64_t lda,
                                    const int32_t *row_index, const int32_t *group_offs, int64_t groups,
                                    int64_t rows, const uint8_t *w_codes, const uint8_t *w_scales, int64_t N,
                                    void *c, fp4_dtype ct, int64_t ldc, hipStream_t stream)
{
    bool empty = false;
    FP4_TRY(check_grouped(a_rows, K, row_index, group_offs, groups, rows, N, 128, c, ct, ldc, &empty));
    if (empty) return FP4_OK;
    FP4_TRY(check_matrix(a, a_rows, K, lda, 2));
    FP4_TRY(check_grouped_limits(a_rows, K, lda, false, groups, rows, N));
    FP4_TRY(check_packed(w_codes, w_scales));
    FP4_TRY(check_device());
    NvGemmArgs g = grouped_args(a_rows, K, row_index, group_offs, groups, rows, w_codes, w_scales, nullptr, N, c,
                                ct, ldc);
    g.a = reinterpret_cast<const uint16_t *>(a);
    g.lda = lda;
    return launch_grouped_gemm(g, 2, stream);
}

fp4_status nvfp4_grouped_gemm_w4a4_prequant(const uint8_t *a_codes, const uint8_t *a_scales,
                                            const float *a_tscale, int64_t a_rows, int64_t K,
                                            const int32_t *row_index, const int32_t *group_offs,
                                            int64_t groups, int64_t rows, const uint8_t *w_codes,
                                            const uint8_t *w_scales, const float *w_tscale, int64_t N,
                                            void *c, fp4_dtype ct, int64_t ldc, hipStream_t stream)
{
    bool empty = false;
    FP4_TRY(check_grouped(a_rows, K, row_index, group_offs, groups, rows, N, 64, c, ct, ldc, &empty));
    if (empty) return FP4_OK;
    FP4_TRY(check_grouped_limits(a_rows, K, K, true, groups, rows, N));
    FP4_TRY(check_packed(a_codes, a_scales));
    FP4_TRY(check_packed(w_codes, w_scales));
    if (!a_tscale || !w_tscale) return FP4_ERR_NULL;
    FP4_TRY(check_device());
    NvGemmArgs g = grouped_args(a_rows, K, row_index, group_offs, groups, rows, w_codes, w_scales, w_tscale, N, c,
                                ct, ldc);
    g.a_codes = a_codes;
    g.a_scales = a_scales;
    g.a_tscale = a_tscale;
    g.a_per_row = 1;
    return launch_grouped_gemm(g, 1, stream);
}

size_t nvfp4_grouped_gemm_w4a4_workspace(int64_t a_rows, int64_t K)
{
    return gemm_w4a4_workspace(a_rows, K, FP4_SCALE_PER_ROW);
}

fp4_status nvfp4_grouped_gemm_w4a4(const void *a, int64_t a_rows, int64_t K, int64_t lda,
                                   const int32_t *row_index, const int32_t *group_offs, int64_t groups,
                                   int64_t rows, const uint8_t *w_codes, const uint8_t *w_scales,
                                   const float *w_tscale, int64_t N, void *c, fp4_dtype ct, int64_t ldc, void *ws,
                                   size_t ws_bytes, hipStream_t stream)
{
    bool empty = false;
    FP4_TRY(check_grouped(a_rows, K, row_index, group_offs, groups, rows, N, 64, c, ct, ldc, &empty));
    if (empty) return FP4_OK;
    FP4_TRY(check_matrix(a, a_rows, K, lda, 2));
    if (a_rows * K > kMaxFlatElems) return FP4_ERR_SHAPE;
    FP4_TRY(check_grouped_limits(a_rows, K, lda, true, groups, rows, N));  // before A is quantized
    FP4_TRY(check_packed(w_codes, w_scales));
    if (!w_tscale) return FP4_ERR_NULL;
    if (!ws || !aligned16(ws) || ws_bytes < nvfp4_grouped_gemm_w4a4_workspace(a_rows, K))
        return FP4_ERR_WORKSPACE;
    FP4_TRY(check_device());
    size_t co, so, to;
    gemm_w4a4_workspace_offsets(a_rows, K, &co, &so, &to);
    uint8_t *base = reinterpret_cast<uint8_t *>(ws);
    float *at = reinterpret_cast<float *>(base + to);
    FP4_TRY(launch_nvfp4_quantize(a, FP4_BF16, a_rows, K, lda, base + co, base + so, at, FP4_SCALE_PER_ROW,
                                  nullptr, nullptr, stream));
    return nvfp4_grouped_gemm_w4a4_prequant(base + co, base + so, at, a_rows, K, row_index, group_offs, groups,
                                            rows, w_codes, w_scales, w_tscale, N, c, ct, ldc, stream);
}

}  // extern "C"
