"""GPU parity of the GEMMs with operands at and past their 32-bit offset limits.

W4A16 and W4A4 (aixq.cc article, "Core difference: W4A4 vs W4A16") on NVFP4
(NVFP4 wiki, format section) and MXFP4 (edge-FP4 article, section "FP4 as the
next core standard"), K = 5120:
  - NVFP4 W4A16 and W4A4, A of 209,716 rows (2,147,491,840 bytes of bf16); and
    W4A16 with W of 838,861 rows (2,147,484,160 code bytes).  The ring kernel
    addresses operands with 32-bit byte offsets, so these take the tile kernel
    with 64-bit addressing;
  - MXFP4 W4A4 with A's codes past 2^31 bytes (1,048,576 rows: the staged
    kernel's unsigned 32-bit offsets) and past 2^32 bytes (1,677,722 rows: the
    64-bit tile kernel);
  - the segment-major MXFP4 GEMM and W4A8 just under their 2^31-byte limits
    (838,860 and 419,430 rows), the former also equal bit for bit to the
    row-major kernel.
Operands repeat a seeded base of 679 rows (A: bf16 activation rows; W: the
oracle's quantization of 679 weight rows, so an NVFP4 tensor scale is that of
the whole W), row r being base row r mod 679; 679 does not divide the row
offsets at which a 32-bit byte offset would wrap, so a wrapped read lands on a
different row.  C is compared with the oracle's fp64 product on sampled rows
(or columns) that include those offsets, |err| <= 2e-3 sum_k |a w|.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import assert_gemm_close, bf16bits_to_dev, dev, log
from synthetic import activations_f32, to_bf16_bits, weights

pytestmark = pytest.mark.gpu

K = 5120
P = 679
CHUNK = 65536


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def fp4():
    import block_scaled_fp4_04_amd as m

    return m


def _tile_rows(base_dev, rows):
    """[rows, ...] device tensor whose row r is base_dev[r % P] (built in chunks)."""
    out = torch.empty((rows,) + tuple(base_dev.shape[1:]), dtype=base_dev.dtype, device=dev())
    for r0 in range(0, rows, CHUNK):
        r = torch.arange(r0, min(rows, r0 + CHUNK), device=dev())
        out[r0:r0 + r.numel()] = base_dev[r % P]
    return out


def _sample(n, byte_row_pitch, seed):
    """Rows around every 2^31-byte multiple (up to 2^33) plus the ends and random rows."""
    s = [0, 1, n - 2, n - 1]
    for mult in range(1, 5):
        r = (mult << 31) // byte_row_pitch
        s += [r - 1, r, r + 1]
    rng = np.random.default_rng(seed)
    s = np.unique(np.concatenate([s, rng.choice(n, 10, replace=False)]))
    return s[s < n]


def _a_base():
    return to_bf16_bits(activations_f32(P, K, 0.005, 30.0, seed=41))


def _w_small(N, seed):
    w = to_bf16_bits(weights(N, K, 0.02, 0.001, 20.0, seed=seed))
    return oracle.nvfp4_quantize(w)


def _packed_nv(codes, scales, tscale):
    return fp4().PackedNVFP4(torch.from_numpy(codes).to(dev()), torch.from_numpy(scales).to(dev()),
                             torch.from_numpy(tscale).to(dev()), codes.shape[0], codes.shape[1] * 2)


@pytest.mark.parametrize("kind", ["w4a16", "w4a4"])
def test_nvfp4_gemm_a_past_2gib(kind):
    M, N = 209716, 256
    assert M * K * 2 >= (1 << 31)
    ab = _a_base()
    log(f"gemm_{kind} A {M}x{K} bf16 ({M * K * 2} bytes), N={N}")
    a = _tile_rows(bf16bits_to_dev(ab), M)
    wc, wsc, wt = _w_small(N, seed=43)
    w = _packed_nv(wc, wsc, wt)
    if kind == "w4a16":
        c = fp4().gemm_w4a16(a, w, dtype=torch.float32)
    else:
        c = fp4().gemm_w4a4(a, w, a_mode="row", dtype=torch.float32)
    torch.cuda.synchronize()
    rows = _sample(M, K * 2, seed=44)
    a_rows = ab[rows % P]
    if kind == "w4a16":
        ref, tol = oracle.gemm_w4a16_ref(a_rows, wc, wsc, wt)
    else:
        ref, tol = oracle.gemm_w4a4_ref(a_rows, wc, wsc, wt, a_per_row=True)
    assert_gemm_close(c[torch.from_numpy(rows).to(dev())], ref, tol, f"{kind} A past 2 GiB")
    del a, c
    torch.cuda.empty_cache()


def test_nvfp4_gemm_w_past_2gib():
    M, N = 64, 838861
    assert N * K // 2 >= (1 << 31)
    a = to_bf16_bits(activations_f32(M, K, 0.005, 30.0, seed=45))
    wc, wsc, wt = _w_small(P, seed=46)        # the base rows; the tensor scale is W's
    log(f"gemm_w4a16 W {N}x{K} NVFP4 ({N * K // 2} code bytes), M={M}")
    codes = _tile_rows(torch.from_numpy(wc).to(dev()), N)
    scales = _tile_rows(torch.from_numpy(wsc).to(dev()), N)
    w = fp4().PackedNVFP4(codes, scales, torch.from_numpy(wt).to(dev()), N, K)
    c = fp4().gemm_w4a16(bf16bits_to_dev(a), w, dtype=torch.float32)
    torch.cuda.synchronize()
    cols = _sample(N, K // 2, seed=47)
    ref, tol = oracle.gemm_w4a16_ref(a, wc[cols % P], wsc[cols % P], wt)
    assert_gemm_close(c[:, torch.from_numpy(cols).to(dev())], ref, tol, "w4a16 W past 2 GiB")
    del codes, scales, c
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ MXFP4 --
#
# MXFP4 (edge-FP4 article, section "FP4 as the next core standard": E8M0 scale
# per 32).  The row-major W4A4 GEMM runs the staged kernel while A's codes stay
# under 2^32 bytes (unsigned 32-bit offsets) and the 64-bit tile kernel beyond;
# the segment-major kernel and W4A8 (MXFP8 A, one byte a value) take operands up
# to just under 2^31 bytes.

def _w_small_mx(N, seed):
    w = to_bf16_bits(weights(N, K, 0.02, 0.001, 20.0, seed=seed))
    return oracle.mxfp4_quantize(w)


def _mx_rows(M):
    return np.union1d(_sample(M, K // 2, seed=M % 1000), _sample(M, K * 2, seed=M % 997))


@pytest.mark.parametrize("M", [1048576, 1677722])   # A codes past 2^31 (staged kernel), past 2^32 (tile kernel)
def test_mxfp4_gemm_a_past_2gib_and_4gib(M):
    N = 256
    ab = _a_base()
    log(f"mxfp4_gemm_w4a4 A {M}x{K} bf16 ({M * K // 2} bytes of A codes), N={N}")
    a = _tile_rows(bf16bits_to_dev(ab), M)
    wc, wsc = _w_small_mx(N, seed=48)
    wp = fp4().PackedMXFP4(torch.from_numpy(wc).to(dev()), torch.from_numpy(wsc).to(dev()), N, K)
    c = fp4().mxfp4_gemm_w4a4(a, wp, dtype=torch.float32)
    torch.cuda.synchronize()
    rows = _mx_rows(M)
    ref, tol = oracle.mxfp4_gemm_w4a4_ref(ab[rows % P], wc, wsc)
    assert_gemm_close(c[torch.from_numpy(rows).to(dev())], ref, tol, f"mxfp4 w4a4 M={M}")
    del a, c
    torch.cuda.empty_cache()


def test_mxfp4_seg_gemm_just_under_2gib():
    M, N = 838860, 256
    assert M * K // 2 < (1 << 31) <= (M + 1) * K // 2
    ab = _a_base()
    log(f"mxfp4_gemm_w4a4_seg A {M}x{K} ({M * K // 2} bytes of A codes), N={N}")
    a = _tile_rows(bf16bits_to_dev(ab), M)
    wc, wsc = _w_small_mx(N, seed=49)
    wp = fp4().PackedMXFP4(torch.from_numpy(wc).to(dev()), torch.from_numpy(wsc).to(dev()), N, K)
    ws = fp4().mxfp4_gemm_w4a4_seg_workspace(M, K, dev())
    c = fp4().mxfp4_gemm_w4a4_seg(a, fp4().mxfp4_pack_decode(wp), dtype=torch.float32, workspace=ws)
    c_rm = fp4().mxfp4_gemm_w4a4(a, wp, dtype=torch.float32)
    torch.cuda.synchronize()
    rows = _mx_rows(M)
    ref, tol = oracle.mxfp4_gemm_w4a4_ref(ab[rows % P], wc, wsc)
    ri = torch.from_numpy(rows).to(dev())
    assert_gemm_close(c[ri], ref, tol, "mxfp4 seg just under 2 GiB")
    assert torch.equal(c, c_rm), "segment-major and row-major kernels differ"
    del a, c, c_rm, ws
    torch.cuda.empty_cache()


def test_w4a8_gemm_just_under_2gib():
    M, N = 419430, 256
    assert M * K < (1 << 31) <= (M + 1) * K
    ab = _a_base()
    log(f"mxfp4_gemm_w4a8 A {M}x{K} ({M * K} bytes of MXFP8 codes), N={N}")
    a = _tile_rows(bf16bits_to_dev(ab), M)
    wc, wsc = _w_small_mx(N, seed=50)
    wp = fp4().PackedMXFP4(torch.from_numpy(wc).to(dev()), torch.from_numpy(wsc).to(dev()), N, K)
    c = fp4().mxfp4_gemm_w4a8(a, wp, dtype=torch.float32)
    torch.cuda.synchronize()
    rows = np.union1d(_sample(M, K, seed=51), _sample(M, K * 2, seed=52))
    ref, tol = oracle.mxfp4_gemm_w4a8_ref(ab[rows % P], wc, wsc)
    assert_gemm_close(c[torch.from_numpy(rows).to(dev())], ref, tol, "w4a8 just under 2 GiB")
    del a, c
    torch.cuda.empty_cache()
