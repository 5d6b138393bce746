"""GPU parity of the row-major NVFP4 GEMMs with an operand past 2 GiB.

W4A16 and W4A4 (aixq.cc article, "Core difference: W4A4 vs W4A16") on the NVFP4
format (NVFP4 wiki, format section).  The ring kernel addresses its operands
with 32-bit byte offsets; gemm_w4a16 / gemm_w4a4 send larger operands to the
tile kernel with 64-bit addressing.  Three cases, K = 5120:
  - W4A16, A of 209,716 rows (2,147,491,840 bytes of bf16), N = 256;
  - W4A4 (A quantized per row inside the call), the same A;
  - W4A16, W of 838,861 rows (2,147,484,160 code bytes), M = 64.
Operands repeat a seeded base of 679 rows (A: bf16 activation rows; W: the
oracle's NVFP4 quantization of 679 weight rows, so the tensor scale is that of
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
