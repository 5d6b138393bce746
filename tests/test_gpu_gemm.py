"""GPU parity: the quantized GEMMs against the oracle's fp64 product.

Each HIP GEMM result must satisfy |C - C_ref| <= 2e-3 * sum_k |a w| per
element, where C_ref is the fp64 product of the exactly dequantized operands.
Small and ragged shapes (several tiles plus a tail, K not a multiple of the
kernel's step) are checked in full; the workloads at full size are checked on
sampled rows.  When every operand is an E2M1 grid value times one power of two
the fp32 result is exact, so the fp32 output must equal the oracle bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import (assert_bf16_is_rounded, assert_gemm_close, bf16bits_to_dev, dev, f32_to_dev, log,
                     sample_rows)
from synthetic import WORKLOADS, activations_f32, to_bf16_bits, weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def fp4():
    import block_scaled_fp4_04_amd as m

    return m


def _packed_nv(codes, scales, tscale, per_row=False):
    return fp4().PackedNVFP4(torch.from_numpy(codes).to(dev()), torch.from_numpy(scales).to(dev()),
                             torch.from_numpy(tscale).to(dev()), codes.shape[0], codes.shape[1] * 2,
                             per_row)


def _packed_mx(codes, scales):
    return fp4().PackedMXFP4(torch.from_numpy(codes).to(dev()), torch.from_numpy(scales).to(dev()),
                             codes.shape[0], codes.shape[1] * 2)


def _case(M, N, K, seed, a_channels=True):
    w = weights(N, K, 0.02, 0.001, 20.0, seed=seed)
    a = to_bf16_bits(activations_f32(M, K, 0.005 if a_channels else 0.0, 30.0, seed=seed + 1))
    return w, a


SHAPES = [
    # (M, N, K): decode path (M <= 16) and prefill path, ragged in every dim
    (1, 16, 64), (1, 100, 1040), (2, 33, 5120), (4, 517, 5120), (7, 64, 80), (16, 300, 1024),
    (16, 17408, 5120), (17, 260, 1040), (64, 256, 256), (300, 520, 5120), (513, 130, 96),
    (257, 1000, 2048),
    # prefill with K a multiple of 64: one to five 64-wide K stages, ragged M and N
    (40, 70, 64), (300, 300, 128), (257, 513, 192), (513, 260, 320),
    # 258 tiles of 256 x 256: the last 232 columns run as 128 x 128 tiles in a second launch
    (500, 33000, 128),
    # 335 tiles of 256 x 256: the last 3844 columns run as 144 tiles of 128 x 256 (128 x 128
    # tiles would not fit in one round on 256 CUs), ragged in M and N
    (1100, 16900, 256),
]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_w4a16(M, N, K, out):
    log(f"gemm_w4a16 M={M} N={N} K={K} out={out}")
    w, a = _case(M, N, K, seed=M + N + K)
    oc, os_, ot = oracle.nvfp4_quantize(w)
    c = fp4().gemm_w4a16(bf16bits_to_dev(a), _packed_nv(oc, os_, ot),
                         dtype=torch.bfloat16 if out == "bf16" else torch.float32)
    torch.cuda.synchronize()
    ref, tol = oracle.gemm_w4a16_ref(a, oc, os_, ot)
    assert_gemm_close(c, ref, tol, f"w4a16 {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(1, 48, 64), (4, 517, 5120), (16, 300, 1040), (17, 260, 1040),
                                   (300, 520, 5120), (513, 130, 96),
                                   (40, 70, 64), (257, 513, 192), (513, 260, 320), (500, 33000, 128),
                                   (1100, 16900, 256)])
@pytest.mark.parametrize("a_mode", ["row", "tensor"])
def test_w4a4(M, N, K, a_mode):
    log(f"gemm_w4a4 M={M} N={N} K={K} a_mode={a_mode}")
    w, a = _case(M, N, K, seed=3 * M + N + K)
    oc, os_, ot = oracle.nvfp4_quantize(w)
    ws = fp4().gemm_w4a4_workspace(M, K, a_mode)
    c = fp4().gemm_w4a4(bf16bits_to_dev(a), _packed_nv(oc, os_, ot), a_mode=a_mode,
                        dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    # the workspace holds A's NVFP4 form: bit-exact against the oracle
    pa = fp4().w4a4_packed_a(ws, M, K, a_mode)
    ac, asc, ats = oracle.nvfp4_quantize(a, per_row=(a_mode == "row"))
    assert np.array_equal(pa.codes.cpu().numpy(), ac)
    assert np.array_equal(pa.scales.cpu().numpy(), asc)
    assert np.array_equal(pa.tscale.cpu().numpy(), ats)
    ref, tol = oracle.gemm_w4a4_ref(a, oc, os_, ot, a_per_row=(a_mode == "row"))
    assert_gemm_close(c, ref, tol, f"w4a4 {M}x{N}x{K}")
    if K % 128 == 0:
        # W in the decode layout: the same kernel arithmetic, bit for bit
        cs = fp4().gemm_w4a4_seg(bf16bits_to_dev(a), fp4().nvfp4_pack_decode(_packed_nv(oc, os_, ot)),
                                 a_mode=a_mode, dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(cs.view(torch.int32), c.view(torch.int32)), "decode-layout W4A4 differs"


# K % 256 == 0 takes the two-stage kernel (K / 256 odd adds a leading zero stage);
# other K the prefetch kernel with a masked K tail.
@pytest.mark.parametrize("M,N,K", [(1, 32, 64), (5, 100, 96), (16, 300, 1056), (17, 260, 1024),
                                   (300, 520, 5120), (513, 130, 160), (256, 256, 128),
                                   (70, 300, 768), (257, 513, 1280), (9, 40, 256), (1100, 16900, 256)])
@pytest.mark.parametrize("rule", ["ocp", "ceil"])
def test_mxfp4_w4a4(M, N, K, rule):
    log(f"mxfp4_gemm_w4a4 M={M} N={N} K={K} rule={rule}")
    w, a = _case(M, N, K, seed=5 * M + N + K)
    r = oracle.MX_OCP_FLOOR if rule == "ocp" else oracle.MX_CEIL
    wc, wsc = oracle.mxfp4_quantize(to_bf16_bits(w), r)
    ws = torch.empty(fp4().lib().mxfp4_gemm_w4a4_workspace(M, K), dtype=torch.uint8, device=dev())
    c = fp4().mxfp4_gemm_w4a4(bf16bits_to_dev(a), _packed_mx(wc, wsc), rule=rule,
                              dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    pa = fp4().mxfp4_packed_a(ws, M, K, N)
    ac, asc = oracle.mxfp4_quantize(a, r)
    if K % 128 == 0:  # the workspace holds A segment-major: [K/128][M][64] and [K/128][M][4]
        assert pa.codes.shape == (K // 128, M, 64)
        ac = ac.reshape(M, K // 128, 64).transpose(1, 0, 2)
        asc = asc.reshape(M, K // 128, 4).transpose(1, 0, 2)
    assert np.array_equal(pa.codes.cpu().numpy(), ac) and np.array_equal(pa.scales.cpu().numpy(), asc)
    ref, tol = oracle.mxfp4_gemm_w4a4_ref(a, wc, wsc, r)
    assert_gemm_close(c, ref, tol, f"mxfp4 {M}x{N}x{K}")


# ------------------------------------------------------ exact closed form --

def _grid_vals(rng, shape, top_every):
    g = rng.integers(0, 16, shape).astype(np.uint8)
    g[..., ::top_every] = (g[..., ::top_every] & 8) | 7
    mag = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    return np.where(g & 8, -1.0, 1.0) * mag[g & 7]


@pytest.mark.parametrize("M,N,K", [(4, 64, 512), (300, 260, 1024), (16, 520, 5120), (100, 300, 5120)])
def test_w4a16_exact_when_operands_are_grid_values(M, N, K):
    """W = grid * 448 * 2^-9 (tensor scale 2^-9, block bytes 0x7E), A = grid * 4:
    every product is 448 * n with |n| <= 144, partial sums stay below 2^23 * 7 * 64,
    so they are exact in fp32 in any order and fp32 C must equal fp64 C."""
    rng = np.random.default_rng(M + N + K)
    wv = (_grid_vals(rng, (N, K), 16) * 448 * 2.0 ** -9).astype(np.float32)
    av = (_grid_vals(rng, (M, K), 10 ** 9) * 4.0).astype(np.float32)
    oc, os_, ot = oracle.nvfp4_quantize(wv)
    assert ot[0] == 2.0 ** -9 and np.all(os_ == 0x7E)
    a = to_bf16_bits(av)
    c = fp4().gemm_w4a16(bf16bits_to_dev(a), _packed_nv(oc, os_, ot), dtype=torch.float32)
    torch.cuda.synchronize()
    ref, _ = oracle.gemm_w4a16_ref(a, oc, os_, ot)
    assert np.array_equal(c.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("M,N,K", [(4, 64, 512), (300, 260, 1024), (16, 520, 1024)])
def test_w4a4_exact_when_operands_are_grid_values(M, N, K):
    """Both operands grid * 448 * 2^j with a +-6 in every 16-block: quantizing them
    (A per row) reproduces them, products are 448^2 * n / 4, and for K <= 1024 the
    partial sums stay below 2^24 units, so fp32 C must equal fp64 C."""
    rng = np.random.default_rng(M * N + K)
    wv = (_grid_vals(rng, (N, K), 16) * 448 * 2.0 ** -9).astype(np.float32)
    av = (_grid_vals(rng, (M, K), 16) * 448 * 2.0 ** -7).astype(np.float32)
    oc, os_, ot = oracle.nvfp4_quantize(wv)
    a = to_bf16_bits(av)
    ac, asc, ats = oracle.nvfp4_quantize(a, per_row=True)
    assert np.all(ats == np.float32(2.0 ** -7)) and np.all(asc == 0x7E)
    c4 = fp4().gemm_w4a4(bf16bits_to_dev(a), _packed_nv(oc, os_, ot), a_mode="row", dtype=torch.float32)
    torch.cuda.synchronize()
    ref4, _ = oracle.gemm_w4a4_ref(a, oc, os_, ot, a_per_row=True)
    assert np.array_equal(c4.cpu().numpy().astype(np.float64), ref4)


@pytest.mark.parametrize("M,N,K", [(32, 64, 256), (300, 260, 1024), (40, 300, 768)])
def test_mxfp4_exact_when_scales_are_powers_of_two(M, N, K):
    rng = np.random.default_rng(K)
    av = _grid_vals(rng, (M, K), 32).astype(np.float32) * np.float32(2.0 ** 3)
    wv = _grid_vals(rng, (N, K), 32).astype(np.float32) * np.float32(2.0 ** -5)
    wc, wsc = oracle.mxfp4_quantize(wv)
    a = to_bf16_bits(av)
    c = fp4().mxfp4_gemm_w4a4(bf16bits_to_dev(a), _packed_mx(wc, wsc), dtype=torch.float32)
    torch.cuda.synchronize()
    ref, _ = oracle.mxfp4_gemm_w4a4_ref(a, wc, wsc)
    assert np.array_equal(c.cpu().numpy().astype(np.float64), ref)


# --------------------------------------------------------- guard bands ----

def test_output_guard_band_and_determinism():
    M, N, K = 300, 260, 1024
    w, a = _case(M, N, K, seed=99)
    oc, os_, ot = oracle.nvfp4_quantize(w)
    wp = _packed_nv(oc, os_, ot)
    ad = bf16bits_to_dev(a)
    big = torch.full((M + 3, N + 40), -7.0, dtype=torch.float32, device=dev())
    view = big[:M, :N]
    fp4().gemm_w4a16(ad, wp, out=view)
    again = fp4().gemm_w4a16(ad, wp, dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.all(big[:M, N:] == -7.0) and torch.all(big[M:, :] == -7.0)
    assert torch.equal(view, again)
    for dec_m in (1, 16):
        c1 = fp4().gemm_w4a16(ad[:dec_m], wp, dtype=torch.float32)
        c2 = fp4().gemm_w4a16(ad[:dec_m], wp, dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(c1, c2)


# ------------------------------------------------- full-size workloads ----

_cache = {}


def _full_weights():
    if "w" not in _cache:
        wl = WORKLOADS["decode_gemv_k5120_n17408"]
        w = wl.weights()
        _cache["w"] = w
        _cache["nv"] = oracle.nvfp4_quantize(w)
    return _cache["w"], _cache["nv"]


@pytest.mark.parametrize("M", [1, 4, 16])
def test_decode_gemv_full_size(M):
    """fp32 output, every element under 2e-3 * sum|a w|; the bf16 output (the form
    the benchmark times) is that result rounded to nearest even, element for element."""
    wl = WORKLOADS["decode_gemv_k5120_n17408"]
    log(f"decode GEMV full size M={M} N=17408 K=5120")
    _, (oc, os_, ot) = _full_weights()
    a = wl.activations_bf16(M)
    w = _packed_nv(oc, os_, ot)
    c = fp4().gemm_w4a16(bf16bits_to_dev(a), w, dtype=torch.float32)
    cb = fp4().gemm_w4a16(bf16bits_to_dev(a), w, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref, tol = oracle.gemm_w4a16_ref(a, oc, os_, ot)
    assert_gemm_close(c, ref, tol, f"decode M={M}")
    assert_bf16_is_rounded(cb, c, f"decode M={M} bf16")


def _full_size_check(c32, cb, ref_fn, rows, what):
    """c32 / cb: the fp32 and bf16 outputs of one call on the full workload.  The
    sampled rows of c32 against the oracle under the literal bound; all of cb
    against c32 rounded to bf16."""
    ref, tol = ref_fn(rows)
    assert_gemm_close(c32[torch.from_numpy(rows).to(dev())], ref, tol, what)
    assert_bf16_is_rounded(cb, c32, what + " bf16")


def test_prefill_w4a16_full_size_sampled():
    wl = WORKLOADS["prefill_w4a16_m4096"]
    log("prefill W4A16 full size M=4096 N=17408 K=5120 (256 sampled rows vs oracle)")
    _, (oc, os_, ot) = _full_weights()
    a = wl.activations_bf16(4096)
    ad, w = bf16bits_to_dev(a), _packed_nv(oc, os_, ot)
    c = fp4().gemm_w4a16(ad, w, dtype=torch.float32)
    cb = fp4().gemm_w4a16(ad, w, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    _full_size_check(c, cb, lambda r: oracle.gemm_w4a16_ref(a, oc, os_, ot, rows=r), sample_rows(4096),
                     "prefill w4a16 sampled")


def test_prefill_w4a4_full_size_sampled():
    wl = WORKLOADS["prefill_w4a4_m4096"]
    log("prefill W4A4 full size M=4096 N=17408 K=5120 (256 sampled rows vs oracle)")
    _, (oc, os_, ot) = _full_weights()
    a = wl.activations_bf16(4096)
    ad, w = bf16bits_to_dev(a), _packed_nv(oc, os_, ot)
    c = fp4().gemm_w4a4(ad, w, a_mode="row", dtype=torch.float32)
    cb = fp4().gemm_w4a4(ad, w, a_mode="row", dtype=torch.bfloat16)
    torch.cuda.synchronize()
    _full_size_check(c, cb, lambda r: oracle.gemm_w4a4_ref(a, oc, os_, ot, a_per_row=True, rows=r),
                     sample_rows(4096, seed=1), "prefill w4a4 sampled")


def test_mx_vs_nv_full_size_sampled():
    wl = WORKLOADS["mx_vs_nv_w4a4_m8192"]
    log("MXFP4 vs NVFP4 W4A4 full size M=8192 N=17408 K=5120 (256 sampled rows vs oracle)")
    w, _ = _full_weights()
    wb = to_bf16_bits(w)
    a = wl.activations_bf16(8192)
    ad = bf16bits_to_dev(a)
    rows = sample_rows(8192, seed=2)
    wc, wsc = oracle.mxfp4_quantize(wb)
    wm = _packed_mx(wc, wsc)
    cm = fp4().mxfp4_gemm_w4a4(ad, wm, dtype=torch.float32)
    cmb = fp4().mxfp4_gemm_w4a4(ad, wm, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    _full_size_check(cm, cmb, lambda r: oracle.mxfp4_gemm_w4a4_ref(a, wc, wsc, rows=r), rows, "mxfp4 sampled")
    del cm, cmb
    nc, ns, nt = oracle.nvfp4_quantize(wb)
    wn = _packed_nv(nc, ns, nt)
    cn = fp4().gemm_w4a4(ad, wn, a_mode="row", dtype=torch.float32)
    cnb = fp4().gemm_w4a4(ad, wn, a_mode="row", dtype=torch.bfloat16)
    torch.cuda.synchronize()
    _full_size_check(cn, cnb, lambda r: oracle.gemm_w4a4_ref(a, nc, ns, nt, a_per_row=True, rows=r), rows,
                     "nvfp4 w4a4 sampled")


@pytest.mark.parametrize("entry", ["w4a16", "w4a4", "w4a16_decode", "mxfp4_w4a4", "mxfp4_seg"])
def test_split_launch_guard_band(entry):
    """1100 x 16900 x 256 runs as two launches (the last columns on smaller tiles,
    written at a column offset of the output): into a view of a larger bf16 buffer,
    nothing outside the view changes and the view equals the same call's output
    into a tensor of its own."""
    M, N, K = 1100, 16900, 256
    log(f"split launch guard band {entry}")
    w, a = _case(M, N, K, seed=1234)
    ad = bf16bits_to_dev(a)
    if entry.startswith("mxfp4"):
        wc, wsc = oracle.mxfp4_quantize(to_bf16_bits(w))
        wp = _packed_mx(wc, wsc)
        if entry == "mxfp4_seg":
            wd = fp4().mxfp4_pack_decode(wp)
            call = lambda out: fp4().mxfp4_gemm_w4a4_seg(ad, wd, out=out)
        else:
            call = lambda out: fp4().mxfp4_gemm_w4a4(ad, wp, out=out)
    else:
        oc, os_, ot = oracle.nvfp4_quantize(w)
        wp = _packed_nv(oc, os_, ot)
        if entry == "w4a16":
            call = lambda out: fp4().gemm_w4a16(ad, wp, out=out)
        elif entry == "w4a16_decode":
            wd = fp4().nvfp4_pack_decode(wp)
            call = lambda out: fp4().gemm_w4a16_decode(ad, wd, out=out)
        else:
            call = lambda out: fp4().gemm_w4a4(ad, wp, a_mode="row", out=out)
    big = torch.full((M + 3, N + 40), -7.0, dtype=torch.bfloat16, device=dev())
    view = big[:M, :N]
    call(view)
    own = torch.empty(M, N, dtype=torch.bfloat16, device=dev())
    call(own)
    torch.cuda.synchronize()
    assert torch.all(big[:M, N:] == -7.0) and torch.all(big[M:, :] == -7.0)
    assert torch.equal(view.view(torch.int16), own.view(torch.int16))
