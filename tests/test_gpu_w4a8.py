"""GPU parity of W4A8: MXFP8 activations x MXFP4 weights.

W4A8 (edge-FP4 article, eefocus.com: an NPU with native W4A8, weights quantized
to FP4 and activations to FP8), with both operands in OCP MX form.
mxfp8_quantize must equal the oracle byte for byte (codes and E8M0 scales, both
scale rules, bf16 and fp32 inputs, zero blocks, signed zeros, tiny and saturating
blocks); mxfp4_gemm_w4a8 must leave the oracle's MXFP8 bytes of A in its
workspace and meet |C - C_ref| <= 2e-3 * sum_k |a w| against the oracle's fp64
product; with grid-valued operands fp32 C must equal the oracle exactly.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import assert_bf16_is_rounded, assert_gemm_close, bf16bits_to_dev, dev, f32_to_dev, log, sample_rows
from synthetic import WORKLOADS, activations_f32, to_bf16_bits, weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def fp4():
    import block_scaled_fp4_04_amd as m

    return m


def _packed_mx(codes, scales):
    return fp4().PackedMXFP4(torch.from_numpy(codes).to(dev()), torch.from_numpy(scales).to(dev()),
                             codes.shape[0], codes.shape[1] * 2)


def _special_rows(K, seed):
    x = activations_f32(6, K, 0.0, 1.0, seed=seed)
    x[0, :32] = 0.0                                    # zero block
    x[1, :32] = -0.0                                   # negative zero block
    x[2, 32:64] *= 1e-30                               # tiny block
    x[3, :32] = np.float32(1.9 * 2.0 ** 6)             # block maximum past 448 * 2^k (OCP rule saturates)
    x[4, 5] = -1e-20                                   # rounds to a signed zero inside a normal block
    x[5, :32] *= 1e20
    return x


@pytest.mark.parametrize("rows,cols", [(1, 32), (7, 96), (300, 1024), (4096, 5120)])
@pytest.mark.parametrize("rule", ["ocp", "ceil"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_mxfp8_quantize_bit_exact(rows, cols, rule, dtype):
    log(f"mxfp8_quantize {rows}x{cols} rule={rule} in={dtype}")
    x = activations_f32(rows, cols, 0.005, 30.0, seed=rows + cols)
    if rows >= 6:
        x[:6] = _special_rows(cols, seed=cols)
    r = oracle.MX_OCP_FLOOR if rule == "ocp" else oracle.MX_CEIL
    src = to_bf16_bits(x) if dtype == "bf16" else x
    want_c, want_s = oracle.mxfp8_quantize(src, r)
    t = bf16bits_to_dev(src) if dtype == "bf16" else f32_to_dev(x)
    got = fp4().mxfp8_quantize(t, rule=rule)
    torch.cuda.synchronize()
    assert np.array_equal(got.scales.cpu().numpy(), want_s)
    assert np.array_equal(got.codes.cpu().numpy(), want_c)


def _case(M, N, K, seed):
    w = weights(N, K, 0.02, 0.001, 20.0, seed=seed)
    a = to_bf16_bits(activations_f32(M, K, 0.005, 30.0, seed=seed + 1))
    wc, wsc = oracle.mxfp4_quantize(w)
    return a, wc, wsc


SHAPES = [(1, 16, 128), (5, 100, 256), (40, 70, 128), (300, 520, 5120), (257, 513, 1280), (513, 260, 640),
          (16, 300, 1024), (260, 33, 384)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("rule", ["ocp", "ceil"])
def test_w4a8_gemm(M, N, K, rule):
    log(f"mxfp4_gemm_w4a8 M={M} N={N} K={K} rule={rule}")
    a, wc, wsc = _case(M, N, K, seed=5 * M + 3 * N + K)
    r = oracle.MX_OCP_FLOOR if rule == "ocp" else oracle.MX_CEIL
    ws = fp4().mxfp4_gemm_w4a8_workspace(M, K, dev())
    wp = _packed_mx(wc, wsc)
    c = fp4().mxfp4_gemm_w4a8(bf16bits_to_dev(a), wp, rule=rule, dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    pa = fp4().mxfp8_packed_a(ws, M, K)
    ac, asc = oracle.mxfp8_quantize(a, r)
    assert np.array_equal(pa.codes.cpu().numpy(), ac) and np.array_equal(pa.scales.cpu().numpy(), asc)
    ref, tol = oracle.mxfp4_gemm_w4a8_ref(a, wc, wsc, r)
    assert_gemm_close(c, ref, tol, f"w4a8 {M}x{N}x{K}")
    # W in the decode (segment-major) layout: the same kernel arithmetic, bit for bit
    cs = fp4().mxfp4_gemm_w4a8_seg(bf16bits_to_dev(a), fp4().mxfp4_pack_decode(wp), rule=rule,
                                   dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(cs, c), "segment-major W differs from row-major W"


@pytest.mark.parametrize("M,N,K", [(40, 300, 256), (300, 260, 1024)])
def test_w4a8_bf16_output(M, N, K):
    a, wc, wsc = _case(M, N, K, seed=M + N)
    c = fp4().mxfp4_gemm_w4a8(bf16bits_to_dev(a), _packed_mx(wc, wsc), dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref, tol = oracle.mxfp4_gemm_w4a8_ref(a, wc, wsc)
    assert_gemm_close(c, ref, tol, f"w4a8 bf16 {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(33, 300, 384), (300, 260, 1024)])
def test_w4a8_prequant_seg_guard_band(M, N, K):
    log(f"mxfp4_gemm_w4a8_prequant_seg M={M} N={N} K={K}")
    a, wc, wsc = _case(M, N, K, seed=2 * M + N)
    ac, asc = oracle.mxfp8_quantize(a)
    pa = fp4().PackedMXFP8(torch.from_numpy(ac).to(dev()), torch.from_numpy(asc).to(dev()), M, K)
    wp = _packed_mx(wc, wsc)
    big = torch.full((M + 3, N + 40), -5.0, dtype=torch.bfloat16, device=dev())
    view = big[:M, :N]
    fp4().mxfp4_gemm_w4a8_prequant_seg(pa, fp4().mxfp4_pack_decode(wp), out=view)
    rm = fp4().mxfp4_gemm_w4a8_prequant(pa, wp, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.all(big[:M, N:] == -5.0) and torch.all(big[M:, :] == -5.0)
    assert torch.equal(view.view(torch.int16), rm.view(torch.int16))
    ref, tol = oracle.mxfp4_gemm_w4a8_ref(a, wc, wsc)
    assert_gemm_close(view, ref, tol, f"w4a8 prequant seg {M}x{N}x{K}")


def _grid_vals(rng, shape):
    g = rng.integers(0, 16, shape).astype(np.uint8)
    g[..., ::32] = (g[..., ::32] & 8) | 7                 # a +-6 in every 32-block
    mag = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    return g, np.where(g & 8, -1.0, 1.0) * mag[g & 7]


@pytest.mark.parametrize("M,N,K", [(4, 64, 512), (300, 260, 1024), (100, 300, 5120)])
def test_w4a8_exact_with_grid_operands(M, N, K):
    """A: E2M1 grid values with a +-6 in every block, which MXFP8 represents
    exactly (6 * 2^6 = 384 is E4M3); W: grid codes with E8M0 bytes 125..129.
    Every product is a multiple of 2^-4 of magnitude <= 144, so fp32 sums over
    K <= 5120 are exact and fp32 C must equal the oracle's fp64 C."""
    rng = np.random.default_rng(M + 11 * N + K)
    g, _ = _grid_vals(rng, (N, K))
    wc = (g[:, 0::2] | (g[:, 1::2] << 4)).astype(np.uint8)
    wsc = rng.integers(125, 130, size=(N, K // 32)).astype(np.uint8)
    _, av = _grid_vals(rng, (M, K))
    a = to_bf16_bits(av.astype(np.float32))
    c = fp4().mxfp4_gemm_w4a8(bf16bits_to_dev(a), _packed_mx(wc, wsc), dtype=torch.float32)
    torch.cuda.synchronize()
    ref, _ = oracle.mxfp4_gemm_w4a8_ref(a, wc, wsc)
    assert np.array_equal(c.cpu().numpy().astype(np.float64), ref)


def test_w4a8_full_size_sampled():
    wl = WORKLOADS["mx_vs_nv_w4a4_m8192"]
    log("W4A8 full size M=8192 N=17408 K=5120 (256 sampled rows vs oracle)")
    w = WORKLOADS["decode_gemv_k5120_n17408"].weights()
    wc, wsc = oracle.mxfp4_quantize(to_bf16_bits(w))
    a = wl.activations_bf16(8192)
    wp = _packed_mx(wc, wsc)
    ad = bf16bits_to_dev(a)
    c = fp4().mxfp4_gemm_w4a8(ad, wp, dtype=torch.float32)
    cs = fp4().mxfp4_gemm_w4a8_seg(ad, fp4().mxfp4_pack_decode(wp), dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(cs, c)
    del cs
    cb = fp4().mxfp4_gemm_w4a8(ad, wp, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert_bf16_is_rounded(cb, c, "w4a8 full size")
    rows = sample_rows(8192, seed=4)
    ref, tol = oracle.mxfp4_gemm_w4a8_ref(a, wc, wsc, rows=rows)
    assert_gemm_close(c[torch.from_numpy(rows).to(dev())], ref, tol, "w4a8 sampled")
