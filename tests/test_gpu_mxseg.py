"""GPU parity of the MXFP4 W4A4 GEMM on segment-major operands.

MXFP4 (edge-FP4 article, eefocus.com, section "FP4 as the next core standard"):
E2M1 elements, one E8M0 power-of-two scale per 32 elements.  mxfp4_gemm_w4a4_seg
takes W in the decode layout that mxfp4_pack_decode writes (codes
[K/128][N][64], scales [K/128][N][4]) and quantizes A into its workspace in the
same layout.  Checks:
  - the workspace's A equals the oracle's MXFP4 quantization of A rearranged by
    the layout's definition (a numpy reshape), bit for bit;
  - C meets |C - C_ref| <= 2e-3 * sum_k |a w| against the oracle's fp64 product;
  - C equals mxfp4_gemm_w4a4 on the row-major W (the same kernel reading W
    row-major) and mxfp4_gemm_prequant on row-major A and W (the two-stage
    row-major kernel) bit for bit: the kernels contract the same 64-element K
    steps in the same order;
  - with grid-valued operands and power-of-two scales the fp32 C equals the
    oracle exactly;
  - at the full M = 8192, N = 17408, K = 5120 workload: equal to the row-major
    kernel everywhere and to the oracle on sampled rows.
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


def _seg(codes, scales):
    """The segment-major layout by its definition: byte (s rows + r) 64 + b = codes[r][64 s + b]."""
    rows, nseg = codes.shape[0], codes.shape[1] // 64
    return (np.ascontiguousarray(codes.reshape(rows, nseg, 64).transpose(1, 0, 2)),
            np.ascontiguousarray(scales.reshape(rows, nseg, 4).transpose(1, 0, 2)))


def _case(M, N, K, seed):
    w = weights(N, K, 0.02, 0.001, 20.0, seed=seed)
    a = to_bf16_bits(activations_f32(M, K, 0.005, 30.0, seed=seed + 1))
    return a, w


# one to many 256 x 256 tiles, ragged M and N; K = 1..40 segments, so 0..3
# leading zero slots fill the ring of four
SHAPES = [(1, 32, 128), (5, 100, 384), (16, 300, 1152), (17, 260, 1024), (70, 300, 768),
          (256, 256, 128), (257, 513, 1280), (513, 130, 640), (300, 520, 5120), (40, 1000, 2688),
          # 335 tiles of 256 x 256 on 256 CUs: the last 3844 columns run as 155 tiles of
          # 256 x 128 in a second launch
          (1100, 16900, 256)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("rule", ["ocp", "ceil"])
def test_mxfp4_seg_gemm(M, N, K, rule):
    log(f"mxfp4_gemm_w4a4_seg M={M} N={N} K={K} rule={rule}")
    a, w = _case(M, N, K, seed=7 * M + N + K)
    r = oracle.MX_OCP_FLOOR if rule == "ocp" else oracle.MX_CEIL
    wc, wsc = oracle.mxfp4_quantize(to_bf16_bits(w), r)
    wp = _packed_mx(wc, wsc)
    wd = fp4().mxfp4_pack_decode(wp)
    ad = bf16bits_to_dev(a)
    ws = fp4().mxfp4_gemm_w4a4_seg_workspace(M, K, dev())
    c = fp4().mxfp4_gemm_w4a4_seg(ad, wd, rule=rule, dtype=torch.float32, workspace=ws)
    c_rm = fp4().mxfp4_gemm_w4a4(ad, wp, rule=rule, dtype=torch.float32)
    torch.cuda.synchronize()
    pa = fp4().mxfp4_seg_packed_a(ws, M, K)
    ac, asc = oracle.mxfp4_quantize(a, r)
    acp, asp = _seg(ac, asc)
    assert np.array_equal(pa.codes.cpu().numpy(), acp) and np.array_equal(pa.scales.cpu().numpy(), asp)
    ref, tol = oracle.mxfp4_gemm_w4a4_ref(a, wc, wsc, r)
    assert_gemm_close(c, ref, tol, f"mxfp4 seg {M}x{N}x{K}")
    assert torch.equal(c, c_rm), "segment-major and row-major kernels differ"
    c_2s = fp4().mxfp4_gemm_prequant(_packed_mx(ac, asc), wp, dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(c, c_2s), "segment kernel and two-stage row-major kernel differ"


@pytest.mark.parametrize("M,N,K", [(33, 300, 640), (300, 260, 1024)])
def test_mxfp4_seg_prequant_bf16_and_guard_band(M, N, K):
    log(f"mxfp4_gemm_prequant_seg bf16 M={M} N={N} K={K}")
    a, w = _case(M, N, K, seed=M + 5 * N + K)
    wc, wsc = oracle.mxfp4_quantize(to_bf16_bits(w))
    ac, asc = oracle.mxfp4_quantize(a)
    wd = fp4().mxfp4_pack_decode(_packed_mx(wc, wsc))
    ad = fp4().mxfp4_pack_decode(_packed_mx(ac, asc))  # the layout applies to any MXFP4 matrix
    big = torch.full((M + 3, N + 40), -7.0, dtype=torch.bfloat16, device=dev())
    view = big[:M, :N]
    fp4().mxfp4_gemm_prequant_seg(ad, wd, out=view)
    rm = fp4().mxfp4_gemm_prequant(_packed_mx(ac, asc), _packed_mx(wc, wsc), dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.all(big[:M, N:] == -7.0) and torch.all(big[M:, :] == -7.0)
    assert torch.equal(view.view(torch.int16), rm.view(torch.int16))
    ref, tol = oracle.mxfp4_gemm_w4a4_ref(a, wc, wsc)
    assert_gemm_close(view, ref, tol, f"mxfp4 seg prequant {M}x{N}x{K}")


def _grid_vals(rng, shape, top_every):
    g = rng.integers(0, 16, shape).astype(np.uint8)
    g[..., ::top_every] = (g[..., ::top_every] & 8) | 7
    mag = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    return np.where(g & 8, -1.0, 1.0) * mag[g & 7]


@pytest.mark.parametrize("M,N,K", [(32, 64, 256), (300, 260, 1152), (40, 300, 384)])
def test_mxfp4_seg_exact_when_scales_are_powers_of_two(M, N, K):
    rng = np.random.default_rng(K + M)
    av = _grid_vals(rng, (M, K), 32).astype(np.float32) * np.float32(2.0 ** 3)
    wv = _grid_vals(rng, (N, K), 32).astype(np.float32) * np.float32(2.0 ** -5)
    wc, wsc = oracle.mxfp4_quantize(wv)
    a = to_bf16_bits(av)
    c = fp4().mxfp4_gemm_w4a4_seg(bf16bits_to_dev(a), fp4().mxfp4_pack_decode(_packed_mx(wc, wsc)),
                                  dtype=torch.float32)
    torch.cuda.synchronize()
    ref, _ = oracle.mxfp4_gemm_w4a4_ref(a, wc, wsc)
    assert np.array_equal(c.cpu().numpy().astype(np.float64), ref)


def test_mxfp4_seg_full_size():
    wl = WORKLOADS["mx_vs_nv_w4a4_m8192"]
    M, N, K = 8192, wl.N, wl.K
    log(f"mxfp4_gemm_w4a4_seg full size M={M} N={N} K={K} (all of C vs the row-major kernel, 256 sampled rows vs oracle)")
    w = WORKLOADS["decode_gemv_k5120_n17408"].weights()
    wb = to_bf16_bits(w)
    a = wl.activations_bf16(M)
    wc, wsc = oracle.mxfp4_quantize(wb)
    wp = _packed_mx(wc, wsc)
    wd = fp4().mxfp4_pack_decode(wp)
    ad = bf16bits_to_dev(a)
    cs = fp4().mxfp4_gemm_w4a4_seg(ad, wd, dtype=torch.float32)
    cr = fp4().mxfp4_gemm_w4a4(ad, wp, dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(cs, cr)
    del cr
    csb = fp4().mxfp4_gemm_w4a4_seg(ad, wd, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert_bf16_is_rounded(csb, cs, "mxfp4 seg full size")
    rows = sample_rows(M, seed=4)
    ref, tol = oracle.mxfp4_gemm_w4a4_ref(a, wc, wsc, rows=rows)
    assert_gemm_close(cs[torch.from_numpy(rows).to(dev())], ref, tol, "mxfp4 seg full size sampled")
