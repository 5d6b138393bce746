"""Pins for the oracle's GEMM references (CPU only).

W4A16 multiplies dequantized 4-bit weights by 16-bit activations; W4A4
quantizes the activations too (Unsloth Dynamic NVFP4 article, aixq.cc, section
"Core difference: W4A4 vs W4A16").  Pins: exact integer arithmetic when every
operand is an E2M1 grid value times one power of two, the C triple loop against
numpy's float64 matmul, and single-product enumeration.
"""
import numpy as np
import pytest

from synthetic import weights, to_bf16_bits

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _grid_value(c):
    c = np.asarray(c)
    return np.where(c & 8, -1.0, 1.0) * GRID[c & 7]


def _unpack(codes):
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = codes & 15
    out[..., 1::2] = codes >> 4
    return out


def _grid_operand(rng, rows, cols, scale_pow, force_top=True):
    g = rng.integers(0, 16, (rows, cols)).astype(np.uint8)
    if force_top:
        g[:, ::16] = (g[:, ::16] & 8) | 7
    return g, _grid_value(g) * 2.0 ** scale_pow


@pytest.mark.parametrize("M,N,K", [(4, 8, 64), (3, 5, 256), (16, 16, 1024)])
def test_w4a16_closed_form_exact(oracle_mod, M, N, K):
    """W = grid * 2^j with every block scale equal; A = grid * 2^i in bf16.  Every
    product is an integer multiple of 0.25 * 2^(i+j), so the result is an exact
    integer computation."""
    rng = np.random.default_rng(M * N + K)
    gw, wv = _grid_operand(rng, N, K, -3)
    ga, av = _grid_operand(rng, M, K, 2, force_top=False)
    # W quantizes back to itself: amax = 6 * 2^-3 in every block -> tensor scale
    # 6*2^-3/2688, block scale 448 (0x7E) everywhere.
    codes, scales, ts = oracle_mod.nvfp4_quantize(wv.astype(np.float32))
    assert np.all(scales == 0x7E) and np.array_equal(_unpack(codes), gw)
    a_bf16 = to_bf16_bits(av.astype(np.float32))
    c, t = oracle_mod.gemm_w4a16_ref(a_bf16, codes, scales, ts)
    # exact: every dequantized weight is g_w * 448 * ts (block byte 0x7E) and
    # every activation is g_a * 2^2; with integers (2 g_a)(2 g_w) the sum is an
    # integer times 0.25 * 2^2 * 448 * ts, exact in fp64 in any order
    ia = (2 * _grid_value(ga)).astype(np.int64)
    iw = (2 * _grid_value(gw)).astype(np.int64)
    s = np.float64(ts[0]) * 448.0
    exact_ts = (ia @ iw.T).astype(np.float64) * 0.25 * 2.0 ** 2 * s
    assert np.array_equal(c, exact_ts)
    assert np.all(t >= np.abs(c))


@pytest.mark.parametrize("M,N,K", [(4, 8, 64), (7, 9, 160)])
def test_w4a16_exact_with_power_of_two_tensor_scale(oracle_mod, M, N, K):
    """Tensor scale a power of two: choose amax = 2688 * 2^j, block scale 448."""
    rng = np.random.default_rng(K)
    gw, _ = _grid_operand(rng, N, K, 0)
    wv = _grid_value(gw) * 448.0 * 2.0 ** -9        # amax = 6*448*2^-9 -> ts = 2^-9
    codes, scales, ts = oracle_mod.nvfp4_quantize(wv.astype(np.float32))
    assert ts[0] == 2.0 ** -9 and np.all(scales == 0x7E)
    ga, av = _grid_operand(rng, M, K, 0, force_top=False)
    c, _ = oracle_mod.gemm_w4a16_ref(to_bf16_bits(av.astype(np.float32)), codes, scales, ts)
    ia = (2 * _grid_value(ga)).astype(np.int64)
    iw = (2 * _grid_value(gw)).astype(np.int64)
    exact = (ia @ iw.T).astype(np.float64) * 0.25 * 448.0 * 2.0 ** -9
    assert np.array_equal(c, exact)


def test_triple_loop_matches_numpy(oracle_mod):
    rng = np.random.default_rng(1)
    a = rng.standard_normal((6, 96))
    w = rng.standard_normal((10, 96))
    c1, t1 = oracle_mod.gemm_f64_loop(a, w)
    c2, t2 = oracle_mod.gemm_f64(a, w)
    assert np.allclose(c1, c2, rtol=1e-12, atol=1e-12)
    assert np.allclose(t1, t2, rtol=1e-12)
    # brute force by Python sums on a few entries
    for m, n in [(0, 0), (5, 9), (3, 4)]:
        assert abs(c1[m, n] - sum(a[m, k] * w[n, k] for k in range(96))) < 1e-12


def test_single_products_enumerated(oracle_mod):
    """One 16-block, one non-zero entry in each operand: the reference is the
    product of the two decoded values, for all 16 x 16 code pairs."""
    for ca in range(16):
        for cw in range(16):
            a = np.zeros((1, 16)); w = np.zeros((1, 16))
            a[0, 5] = _grid_value(ca); w[0, 5] = _grid_value(cw)
            c, t = oracle_mod.gemm_f64_loop(a, w)
            assert c[0, 0] == _grid_value(ca) * _grid_value(cw)
            assert t[0, 0] == abs(c[0, 0])


def test_w4a4_ref_equals_w4a16_ref_when_a_is_representable(oracle_mod):
    """If each row of A is already an NVFP4 tensor (grid x 448 x 2^j per row),
    quantizing it per row reproduces it, so W4A4 and W4A16 references agree."""
    rng = np.random.default_rng(3)
    M, N, K = 5, 7, 128
    ga, _ = _grid_operand(rng, M, K, 0)
    av = _grid_value(ga) * 448.0 * 2.0 ** -4
    a_bf16 = to_bf16_bits(av.astype(np.float32))
    w = weights(N, K, 0.02, 0.01, 20.0, seed=4)
    wc, ws, wt = oracle_mod.nvfp4_quantize(w)
    c16, _ = oracle_mod.gemm_w4a16_ref(a_bf16, wc, ws, wt)
    c4, _ = oracle_mod.gemm_w4a4_ref(a_bf16, wc, ws, wt, a_per_row=True)
    assert np.array_equal(c16, c4)


def test_row_subset(oracle_mod):
    """Restricting the reference to some rows of A gives those rows (up to fp64
    summation order inside the BLAS matmul)."""
    w = weights(9, 64, seed=5)
    wc, ws, wt = oracle_mod.nvfp4_quantize(w)
    a = to_bf16_bits(weights(6, 64, seed=6))
    full, _ = oracle_mod.gemm_w4a16_ref(a, wc, ws, wt)
    part, _ = oracle_mod.gemm_w4a16_ref(a, wc, ws, wt, rows=np.array([1, 4]))
    assert np.allclose(part, full[[1, 4]], rtol=1e-13, atol=1e-300)
    full4, _ = oracle_mod.gemm_w4a4_ref(a, wc, ws, wt)
    part4, _ = oracle_mod.gemm_w4a4_ref(a, wc, ws, wt, rows=np.array([2, 5]))
    assert np.allclose(part4, full4[[2, 5]], rtol=1e-13, atol=1e-300)
    mc, ms = oracle_mod.mxfp4_quantize(w)
    fullm, _ = oracle_mod.mxfp4_gemm_w4a4_ref(a, mc, ms)
    partm, _ = oracle_mod.mxfp4_gemm_w4a4_ref(a, mc, ms, rows=np.array([0, 3]))
    assert np.allclose(partm, fullm[[0, 3]], rtol=1e-13, atol=1e-300)


def test_mxfp4_plain_fp4_matmul_when_scales_are_one(oracle_mod):
    rng = np.random.default_rng(7)
    M, N, K = 4, 6, 64
    ga, av = _grid_operand(rng, M, K, 0, force_top=False)
    gw, wv = _grid_operand(rng, N, K, 0, force_top=False)
    # force each 32-block's amax to 4 or 6 so the OCP scale byte is 127 (2^0)
    ga[:, ::32] = 6; av = _grid_value(ga)
    gw[:, ::32] = 7; wv = _grid_value(gw)
    wc, ws = oracle_mod.mxfp4_quantize(wv.astype(np.float32))
    assert np.all(ws == 127)
    c, _ = oracle_mod.mxfp4_gemm_w4a4_ref(to_bf16_bits(av.astype(np.float32)), wc, ws)
    assert np.array_equal(c, av @ wv.T)


def test_mxfp4_w4a16_ref_brute_force(oracle_mod):
    # independent pin: a triple loop over E2M1 grid values times 2^(byte - 127),
    # written here from the MXFP4 definition, against the oracle's W4A16 reference
    rng = np.random.default_rng(11)
    M, N, K = 3, 5, 64
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = rng.integers(110, 140, size=(N, K // 32), dtype=np.uint8)
    a = to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    w = np.zeros((N, K))
    for n in range(N):
        for k in range(K):
            nib = (int(codes[n, k // 2]) >> (4 * (k % 2))) & 15
            v = grid[nib & 7] * (-1.0 if nib & 8 else 1.0)
            w[n, k] = v * 2.0 ** (int(scales[n, k // 32]) - 127)
    av = (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            ref[m, n] = sum(av[m, k] * w[n, k] for k in range(K))
    got, tol = oracle_mod.mxfp4_gemm_w4a16_ref(a, codes, scales)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-300)
    assert np.all(tol >= np.abs(got) - 1e-300)


def test_mxfp4_w4a8_ref_brute_force(oracle_mod):
    # independent pin: A quantized by the oracle's MXFP8 (pinned on its own), both
    # operands decoded here from the E4M3 / E2M1 / E8M0 definitions, triple loop
    rng = np.random.default_rng(13)
    M, N, K = 3, 4, 64
    a = to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    ac, asc = oracle_mod.mxfp8_quantize(a)
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = rng.integers(120, 135, size=(N, K // 32), dtype=np.uint8)
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]

    def e4m3(b):
        s, e, m = b >> 7, (b >> 3) & 15, b & 7
        v = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        return -v if s else v

    ref = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            t = 0.0
            for k in range(K):
                av = e4m3(int(ac[m, k])) * 2.0 ** (int(asc[m, k // 32]) - 127)
                nib = (int(codes[n, k // 2]) >> (4 * (k % 2))) & 15
                wv = grid[nib & 7] * (-1.0 if nib & 8 else 1.0) * 2.0 ** (int(scales[n, k // 32]) - 127)
                t += av * wv
            ref[m, n] = t
    got, _ = oracle_mod.mxfp4_gemm_w4a8_ref(a, codes, scales)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-300)
