"""GPU parity of the MXFP4 W4A16 paths (weights MXFP4, activations bf16).

MXFP4 (edge-FP4 article, eefocus.com, section "FP4 as the next core standard"):
E2M1 elements, one E8M0 power-of-two scale per 32 elements, no tensor scale.
W4A16 (aixq.cc article, "Core difference: W4A4 vs W4A16"): 16-bit activations.
The prefill GEMM (mxfp4_gemm_w4a16, row-major weights) and the decode GEMV
(mxfp4_gemm_w4a16_decode on the layout mxfp4_pack_decode writes) must meet
|C - C_ref| <= 2e-3 * sum_k |a w| against the oracle's fp64 product of the
exactly dequantized operands; mxfp4_pack_decode must equal a numpy reshape of the
row-major bytes; with grid-valued operands fp32 C must equal the oracle exactly.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import assert_bf16_is_rounded, assert_gemm_close, bf16bits_to_dev, dev, log, sample_rows
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


def _case(M, N, K, seed):
    w = weights(N, K, 0.02, 0.001, 20.0, seed=seed)
    a = to_bf16_bits(activations_f32(M, K, 0.005, 30.0, seed=seed + 1))
    wc, wsc = oracle.mxfp4_quantize(w)
    return a, wc, wsc


# prefill GEMM: one to many 256 x 256 tiles, ragged M and N, K stages 2..80, and a
# grid with a last round that runs as 128 x 128 tiles (500 x 33000)
PREFILL = [(1, 16, 128), (5, 100, 384), (40, 70, 128), (300, 520, 5120), (257, 513, 1280),
           (513, 260, 640), (500, 33000, 128), (16, 300, 1024), (1100, 16900, 256)]


@pytest.mark.parametrize("M,N,K", PREFILL)
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_mxfp4_w4a16(M, N, K, out):
    log(f"mxfp4_gemm_w4a16 M={M} N={N} K={K} out={out}")
    a, wc, wsc = _case(M, N, K, seed=3 * M + N + K)
    c = fp4().mxfp4_gemm_w4a16(bf16bits_to_dev(a), _packed_mx(wc, wsc),
                               dtype=torch.bfloat16 if out == "bf16" else torch.float32)
    torch.cuda.synchronize()
    ref, tol = oracle.mxfp4_gemm_w4a16_ref(a, wc, wsc)
    assert_gemm_close(c, ref, tol, f"mxfp4 w4a16 {M}x{N}x{K}")


def _grid_vals(rng, shape):
    g = rng.integers(0, 16, shape).astype(np.uint8)
    mag = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    return g, np.where(g & 8, -1.0, 1.0) * mag[g & 7]


def _grid_weight(rng, N, K):
    """Random E2M1 codes and E8M0 bytes 125..129: every weight is a grid value
    times 2^-2 .. 2^2, so with grid-valued A every product is a multiple of 2^-4
    of magnitude <= 144, and for K <= 5120 every partial sum is exact in fp32."""
    g, _ = _grid_vals(rng, (N, K))
    codes = (g[:, 0::2] | (g[:, 1::2] << 4)).astype(np.uint8)
    scales = rng.integers(125, 130, size=(N, K // 32)).astype(np.uint8)
    return codes, scales


@pytest.mark.parametrize("M,N,K", [(4, 64, 512), (300, 260, 1024), (100, 300, 5120)])
def test_mxfp4_w4a16_exact_with_grid_operands(M, N, K):
    rng = np.random.default_rng(M + 7 * N + K)
    wc, wsc = _grid_weight(rng, N, K)
    _, av = _grid_vals(rng, (M, K))
    a = to_bf16_bits(av.astype(np.float32))
    c = fp4().mxfp4_gemm_w4a16(bf16bits_to_dev(a), _packed_mx(wc, wsc), dtype=torch.float32)
    torch.cuda.synchronize()
    ref, _ = oracle.mxfp4_gemm_w4a16_ref(a, wc, wsc)
    assert np.array_equal(c.cpu().numpy().astype(np.float64), ref)


# ------------------------------------------------------------------ decode --

@pytest.mark.parametrize("N,K", [(1, 128), (16, 256), (300, 1152), (17408, 5120)])
def test_mxfp4_pack_decode_layout(N, K):
    log(f"mxfp4_pack_decode N={N} K={K}")
    _, wc, wsc = _case(1, N, K, seed=N + 3 * K)
    d = fp4().mxfp4_pack_decode(_packed_mx(wc, wsc))
    torch.cuda.synchronize()
    nseg = K // 128
    cp = np.ascontiguousarray(wc.reshape(N, nseg, 64).transpose(1, 0, 2))
    sp = np.ascontiguousarray(wsc.reshape(N, nseg, 4).transpose(1, 0, 2))
    assert np.array_equal(d.codes.cpu().numpy(), cp)
    assert np.array_equal(d.scales.cpu().numpy(), sp)


DECODE = [(1, 16, 128), (1, 100, 1024), (2, 33, 5120), (4, 517, 5120), (16, 300, 1024), (5, 40, 384),
          (3, 1000, 8192), (1, 4097, 2048), (16, 1, 128), (7, 40000, 256), (16, 2000, 1152),
          (1, 700, 9216), (16, 530, 14336),
          # 3, 4, 6 and 7 16-row tiles per workgroup on a 256-CU part
          (16, 9600, 256), (1, 14400, 256), (5, 22400, 128), (4, 27200, 384)]


@pytest.mark.parametrize("M,N,K", DECODE)
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_mxfp4_decode_gemv(M, N, K, out):
    log(f"mxfp4_gemm_w4a16_decode M={M} N={N} K={K} out={out}")
    a, wc, wsc = _case(M, N, K, seed=11 * M + N + K)
    d = fp4().mxfp4_pack_decode(_packed_mx(wc, wsc))
    c = fp4().mxfp4_gemm_w4a16_decode(bf16bits_to_dev(a), d,
                                      dtype=torch.bfloat16 if out == "bf16" else torch.float32)
    torch.cuda.synchronize()
    ref, tol = oracle.mxfp4_gemm_w4a16_ref(a, wc, wsc)
    assert_gemm_close(c, ref, tol, f"mxfp4 decode {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(1, 64, 512), (4, 520, 5120), (16, 300, 1024)])
def test_mxfp4_decode_exact_with_grid_operands(M, N, K):
    rng = np.random.default_rng(3 * M + N + K)
    wc, wsc = _grid_weight(rng, N, K)
    _, av = _grid_vals(rng, (M, K))
    a = to_bf16_bits(av.astype(np.float32))
    d = fp4().mxfp4_pack_decode(_packed_mx(wc, wsc))
    c = fp4().mxfp4_gemm_w4a16_decode(bf16bits_to_dev(a), d, dtype=torch.float32)
    torch.cuda.synchronize()
    ref, _ = oracle.mxfp4_gemm_w4a16_ref(a, wc, wsc)
    assert np.array_equal(c.cpu().numpy().astype(np.float64), ref)


# M > 16 on the MXFP4 decode layout: the prefill GEMM reading it (a second launch
# of 128 x 128 tiles for the last columns of 500 x 33000)
@pytest.mark.parametrize("M,N,K", [(17, 260, 1024), (40, 70, 128), (300, 520, 5120), (513, 260, 640),
                                   (500, 33000, 128), (1100, 16900, 256)])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_mxfp4_decode_layout_prefill(M, N, K, out):
    log(f"mxfp4_gemm_w4a16_decode (prefill, M > 16) M={M} N={N} K={K} out={out}")
    a, wc, wsc = _case(M, N, K, seed=13 * M + N + K)
    wp = _packed_mx(wc, wsc)
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    ad = bf16bits_to_dev(a)
    c = fp4().mxfp4_gemm_w4a16_decode(ad, fp4().mxfp4_pack_decode(wp), dtype=dt)
    c_rm = fp4().mxfp4_gemm_w4a16(ad, wp, dtype=dt)
    torch.cuda.synchronize()
    ref, tol = oracle.mxfp4_gemm_w4a16_ref(a, wc, wsc)
    assert_gemm_close(c, ref, tol, f"mxfp4 decode layout prefill {M}x{N}x{K}")
    bits = torch.int16 if out == "bf16" else torch.int32
    assert torch.equal(c.view(bits), c_rm.view(bits)), "decode-layout and row-major prefill differ"


_cache = {}


def _full_mx():
    if "mx" not in _cache:
        w = WORKLOADS["decode_gemv_k5120_n17408"].weights()
        _cache["mx"] = oracle.mxfp4_quantize(w)
    return _cache["mx"]


@pytest.mark.parametrize("M", [1, 4, 16])
def test_mxfp4_decode_full_size(M):
    wl = WORKLOADS["decode_gemv_k5120_n17408"]
    log(f"MXFP4 decode GEMV full size M={M} N=17408 K=5120")
    wc, wsc = _full_mx()
    a = wl.activations_bf16(M)
    d = fp4().mxfp4_pack_decode(_packed_mx(wc, wsc))
    ad = bf16bits_to_dev(a)
    c = fp4().mxfp4_gemm_w4a16_decode(ad, d, dtype=torch.float32)
    cb = fp4().mxfp4_gemm_w4a16_decode(ad, d, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref, tol = oracle.mxfp4_gemm_w4a16_ref(a, wc, wsc)
    assert_gemm_close(c, ref, tol, f"mxfp4 decode M={M}")
    assert_bf16_is_rounded(cb, c, f"mxfp4 decode M={M}")


def test_mxfp4_prefill_full_size_sampled():
    wl = WORKLOADS["prefill_w4a16_m4096"]
    log("MXFP4 W4A16 prefill full size M=4096 N=17408 K=5120 (256 sampled rows vs oracle)")
    wc, wsc = _full_mx()
    a = wl.activations_bf16(4096)
    ad, w = bf16bits_to_dev(a), _packed_mx(wc, wsc)
    c = fp4().mxfp4_gemm_w4a16(ad, w, dtype=torch.float32)
    cb = fp4().mxfp4_gemm_w4a16(ad, w, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = sample_rows(4096, seed=2)
    ref, tol = oracle.mxfp4_gemm_w4a16_ref(a, wc, wsc, rows=rows)
    assert_gemm_close(c[torch.from_numpy(rows).to(dev())], ref, tol, "mxfp4 prefill sampled")
    assert_bf16_is_rounded(cb, c, "mxfp4 prefill")
