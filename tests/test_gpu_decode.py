"""GPU parity of the decode layout and the decode GEMV.

nvfp4_pack_decode only reorders bytes: its output must equal, byte for byte, the
segment-major rearrangement of the oracle's row-major codes and scales, written
here with numpy reshapes.  gemm_w4a16_decode must meet the GEMM bound
|C - C_ref| <= 2e-3 * sum_k |a w| against the oracle's fp64 product, over
shapes that cover one and many 16-row tiles, ragged row counts per workgroup,
waves with no K segment (K / 128 < 8), K past 8192 (run in chunks), more workgroups
than CUs, and the full decode workload; with grid-valued operands the fp32
result is exact and must equal the oracle bit for bit.
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


def _packed_nv(codes, scales, tscale):
    return fp4().PackedNVFP4(torch.from_numpy(codes).to(dev()), torch.from_numpy(scales).to(dev()),
                             torch.from_numpy(tscale).to(dev()), codes.shape[0], codes.shape[1] * 2, False)


def _segment_major(codes, scales):
    """codes [N][K/2] -> [K/128][N][64]; scales [N][K/16] -> [K/128][N][8]."""
    N, half = codes.shape
    nseg = half // 64
    cp = codes.reshape(N, nseg, 64).transpose(1, 0, 2)
    sp = scales.reshape(N, nseg, 8).transpose(1, 0, 2)
    return np.ascontiguousarray(cp), np.ascontiguousarray(sp)


@pytest.mark.parametrize("N,K", [(1, 128), (16, 256), (300, 1024), (17408, 5120)])
def test_pack_decode_layout(N, K):
    log(f"nvfp4_pack_decode N={N} K={K}")
    w = weights(N, K, 0.02, 0.001, 20.0, seed=N + K)
    oc, os_, ot = oracle.nvfp4_quantize(w)
    d = fp4().nvfp4_pack_decode(_packed_nv(oc, os_, ot))
    torch.cuda.synchronize()
    cp, sp = _segment_major(oc, os_)
    assert np.array_equal(d.codes.cpu().numpy(), cp)
    assert np.array_equal(d.scales.cpu().numpy(), sp)


SHAPES = [
    (1, 16, 128), (1, 100, 1024), (2, 33, 5120), (4, 517, 5120), (16, 300, 1024), (5, 40, 384),
    (3, 1000, 8192), (1, 4097, 2048), (16, 1, 128), (7, 40000, 256), (16, 2000, 1152),
    # 3, 4, 6 and 7 16-row tiles per workgroup on a 256-CU part
    (16, 9600, 256), (1, 14400, 256), (5, 22400, 128), (4, 27200, 384),
    # K past 8192, in chunks of 8 S segments: 2 chunks of 40 and 32 segments
    # (K = 9216), 2 of 56 (14336), 3 of 48, 48 and 33 (16512)
    (1, 700, 9216), (4, 300, 14336), (16, 530, 14336), (2, 100, 16512), (16, 64, 16512),
]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_decode_gemv(M, N, K, out):
    log(f"gemm_w4a16_decode M={M} N={N} K={K} out={out}")
    w = weights(N, K, 0.02, 0.001, 20.0, seed=7 * M + N + K)
    a = to_bf16_bits(activations_f32(M, K, 0.005, 30.0, seed=M + 2 * N + K))
    oc, os_, ot = oracle.nvfp4_quantize(w)
    d = fp4().nvfp4_pack_decode(_packed_nv(oc, os_, ot))
    c = fp4().gemm_w4a16_decode(bf16bits_to_dev(a), d, dtype=torch.bfloat16 if out == "bf16" else torch.float32)
    torch.cuda.synchronize()
    ref, tol = oracle.gemm_w4a16_ref(a, oc, os_, ot)
    assert_gemm_close(c, ref, tol, f"decode {M}x{N}x{K}")


@pytest.mark.parametrize("M", [1, 4, 16])
def test_decode_infinite_activation_stays_in_its_row(M):
    """An infinite activation of row 0 in the last K segment (K = 1152: nine
    segments, so waves 5-7 of a workgroup own none and read that segment's
    position for nothing): row 0 of C is +-inf where the weight at that K is
    nonzero and NaN where it is zero, exactly as the fp64 product gives, and every
    other row is finite and within the GEMM bound (a wave that multiplied the
    infinity by its zero codes would turn all of row 0 into NaN)."""
    N, K, k0 = 300, 1152, 1100
    log(f"gemm_w4a16_decode M={M} N={N} K={K} with A[0, {k0}] = +inf")
    w = weights(N, K, 0.02, 0.001, 20.0, seed=91 + M)
    a = to_bf16_bits(activations_f32(M, K, 0.005, 30.0, seed=92 + M))
    a[0, k0] = 0x7F80  # +inf in bf16
    oc, os_, ot = oracle.nvfp4_quantize(w)
    d = fp4().nvfp4_pack_decode(_packed_nv(oc, os_, ot))
    with np.errstate(invalid="ignore"):  # inf * 0 in the reference product
        ref, tol = oracle.gemm_w4a16_ref(a, oc, os_, ot)
    assert np.isnan(ref[0]).any() and np.isinf(ref[0]).any()  # both kinds occur
    for dt in (torch.float32, torch.bfloat16):
        c = fp4().gemm_w4a16_decode(bf16bits_to_dev(a), d, dtype=dt)
        torch.cuda.synchronize()
        got = c.float().cpu().numpy().astype(np.float64)
        assert np.array_equal(np.isnan(got[0]), np.isnan(ref[0])), "NaN positions of row 0"
        inf = np.isinf(ref[0])
        assert np.array_equal(np.isinf(got[0]), inf) and np.array_equal(np.sign(got[0][inf]), np.sign(ref[0][inf]))
        if M > 1:
            assert_gemm_close(c[1:], ref[1:], tol[1:], f"decode rows 1.. with inf in row 0, {dt}")


def _grid_vals(rng, shape, top_every):
    """E2M1 grid values with a +-6 every `top_every` elements (so every 16-block of
    the weight gets the same scale byte)."""
    g = rng.integers(0, 16, shape).astype(np.uint8)
    g[..., ::top_every] = (g[..., ::top_every] & 8) | 7
    mag = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    return np.where(g & 8, -1.0, 1.0) * mag[g & 7]


@pytest.mark.parametrize("M,N,K", [(1, 64, 512), (16, 300, 1024), (4, 520, 5120)])
def test_decode_exact_when_operands_are_grid_values(M, N, K):
    """W = grid * 448 * 2^-9 (every block byte 0x7E), A = grid * 4: products are
    448 * n with |n| <= 144 and partial sums stay far below 2^24 units of 448, so
    fp32 C is exact in any summation order and must equal fp64 C."""
    rng = np.random.default_rng(M + N + K)
    wv = (_grid_vals(rng, (N, K), 16) * 448 * 2.0 ** -9).astype(np.float32)
    av = (_grid_vals(rng, (M, K), 10 ** 9) * 4.0).astype(np.float32)
    oc, os_, ot = oracle.nvfp4_quantize(wv)
    assert ot[0] == 2.0 ** -9 and np.all(os_ == 0x7E)
    a = to_bf16_bits(av)
    d = fp4().nvfp4_pack_decode(_packed_nv(oc, os_, ot))
    c = fp4().gemm_w4a16_decode(bf16bits_to_dev(a), d, dtype=torch.float32)
    torch.cuda.synchronize()
    ref, _ = oracle.gemm_w4a16_ref(a, oc, os_, ot)
    assert np.array_equal(c.cpu().numpy().astype(np.float64), ref)


# M > 16 on the decode layout: the prefill GEMM reading it, ragged tiles, K of one
# to forty segments, and a grid whose last round of columns runs as a second
# launch of 128 x 128 tiles (500 x 33000: its weight rows start at row 32768)
PREFILL = [(17, 260, 1024), (40, 70, 128), (300, 520, 5120), (257, 513, 1280), (513, 260, 640),
           (500, 33000, 128), (1100, 16900, 256)]


@pytest.mark.parametrize("M,N,K", PREFILL)
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_decode_layout_prefill(M, N, K, out):
    log(f"gemm_w4a16_decode (prefill, M > 16) M={M} N={N} K={K} out={out}")
    w = weights(N, K, 0.02, 0.001, 20.0, seed=5 * M + N + K)
    a = to_bf16_bits(activations_f32(M, K, 0.005, 30.0, seed=M + 3 * N + K))
    oc, os_, ot = oracle.nvfp4_quantize(w)
    wp = _packed_nv(oc, os_, ot)
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    ad = bf16bits_to_dev(a)
    c = fp4().gemm_w4a16_decode(ad, fp4().nvfp4_pack_decode(wp), dtype=dt)
    c_rm = fp4().gemm_w4a16(ad, wp, dtype=dt)
    torch.cuda.synchronize()
    ref, tol = oracle.gemm_w4a16_ref(a, oc, os_, ot)
    assert_gemm_close(c, ref, tol, f"decode layout prefill {M}x{N}x{K}")
    bits = torch.int16 if out == "bf16" else torch.int32
    assert torch.equal(c.view(bits), c_rm.view(bits)), "decode-layout and row-major prefill differ"


_cache = {}


def test_decode_layout_prefill_full_size():
    wl = WORKLOADS["prefill_w4a16_m4096"]
    M = 4096
    log(f"gemm_w4a16_decode prefill full size M={M} N={wl.N} K={wl.K} (all of C vs row-major, 256 sampled rows vs oracle)")
    if "nv" not in _cache:
        _cache["nv"] = oracle.nvfp4_quantize(WORKLOADS["decode_gemv_k5120_n17408"].weights())
    oc, os_, ot = _cache["nv"]
    a = wl.activations_bf16(M)
    wp = _packed_nv(oc, os_, ot)
    ad = bf16bits_to_dev(a)
    wd = fp4().nvfp4_pack_decode(wp)
    c = fp4().gemm_w4a16_decode(ad, wd, dtype=torch.float32)
    cb = fp4().gemm_w4a16_decode(ad, wd, dtype=torch.bfloat16)
    c_rm = fp4().gemm_w4a16(ad, wp, dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(c, c_rm)
    assert_bf16_is_rounded(cb, c, "decode layout prefill bf16")
    rows = sample_rows(M, seed=9)
    ref, tol = oracle.gemm_w4a16_ref(a, oc, os_, ot, rows=rows)
    assert_gemm_close(c[torch.from_numpy(rows).to(dev())], ref, tol, "decode layout prefill sampled")


@pytest.mark.parametrize("M", [1, 4, 16])
def test_decode_gemv_full_size(M):
    """The benchmark's call (bf16 output) and the same call with fp32 output: the
    fp32 result within 2e-3 * sum|a w| of the oracle in every element, the bf16
    result that value rounded to nearest even."""
    wl = WORKLOADS["decode_gemv_k5120_n17408"]
    log(f"decode GEMV (decode layout) full size M={M} N=17408 K=5120")
    if "nv" not in _cache:
        _cache["nv"] = oracle.nvfp4_quantize(wl.weights())
    oc, os_, ot = _cache["nv"]
    a = wl.activations_bf16(M)
    d = fp4().nvfp4_pack_decode(_packed_nv(oc, os_, ot))
    ad = bf16bits_to_dev(a)
    c = fp4().gemm_w4a16_decode(ad, d, dtype=torch.float32)
    cb = fp4().gemm_w4a16_decode(ad, d, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref, tol = oracle.gemm_w4a16_ref(a, oc, os_, ot)
    assert_gemm_close(c, ref, tol, f"decode layout M={M}")
    assert_bf16_is_rounded(cb, c, f"decode layout M={M}")
    # the row-major path gives the same numbers up to summation order
    c2 = fp4().gemm_w4a16(ad, _packed_nv(oc, os_, ot), dtype=torch.float32)
    torch.cuda.synchronize()
    assert_gemm_close(c2, ref, tol, f"row-major M={M}")


def test_prepared_calls_replay_the_same_launches():
    """fp4.prepare records the library calls of a thunk (checks made once) and
    replays them: the replayed GEMV and W4A4 calls (the latter with a workspace the
    wrapper allocated inside the thunk) give the eager results, call after call,
    and see new contents of the same input tensors."""
    m = fp4()
    N, K = 1000, 1024
    w = weights(N, K, 0.02, 0.001, 20.0, seed=41)
    oc, os_, ot = oracle.nvfp4_quantize(w)
    wp = _packed_nv(oc, os_, ot)
    wd = m.nvfp4_pack_decode(wp)
    a_bits = to_bf16_bits(activations_f32(16, K, seed=42))
    a = bf16bits_to_dev(a_bits)
    out = torch.empty(16, N, dtype=torch.float32, device=dev())
    gemv = m.prepare(lambda: m.gemm_w4a16_decode(a, wd, out=out))
    w4a4 = m.prepare(lambda: m.gemm_w4a4(a, wp, dtype=torch.float32))   # output and workspace made inside
    eager = m.gemm_w4a16_decode(a, wd, dtype=torch.float32)
    eager4 = m.gemm_w4a4(a, wp, dtype=torch.float32)
    torch.cuda.synchronize()
    c4 = w4a4._keep[0]
    for rep in range(3):
        out.zero_()
        c4.zero_()
        gemv()
        w4a4()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}"
        assert torch.equal(c4, eager4), f"replay {rep}"
    a.mul_(-1)                                   # new contents, same memory
    gemv()
    fresh = m.gemm_w4a16_decode(a, wd, dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(out, fresh) and not torch.equal(out, eager)


def test_read_ceiling_runs_and_reads_nothing_back():
    """The measurement kernel reads its buffer and leaves the sink alone (the sink
    is written only when the XOR of all words hits one fixed constant, which this
    buffer's words do not)."""
    log("fp4blk_read_ceiling on 1 MiB + 16 bytes")
    buf = torch.zeros((1 << 20) + 16, dtype=torch.uint8, device=dev())
    sink = torch.zeros(1, dtype=torch.int32, device=dev())
    for grid in (1, 7, 256, 2048):
        fp4().read_ceiling(buf, grid, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
    with pytest.raises(ValueError):
        fp4().read_ceiling(buf[:1000], 16, sink)
