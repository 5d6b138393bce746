"""Pins for the oracle's NVFP4 quantize / dequantize (CPU only).

The scheme is the two-level one of "NVFP4" (newton.com.tw wiki), section
"Technical principle": 16-value micro-blocks with an E4M3 scale each and one
FP32 scale for the tensor, E2M1 elements, about 4.5 bits per value.  The pins
are a hand-worked example, exact round trips of grid-representable tensors,
power-of-two equivariance, sign symmetry, permutation, the amax block, an error
bound and the storage identity; dequantization is checked against an fp64 product
of torch-decoded E4M3 scales and the E2M1 grid.
"""
import json
import os

import numpy as np
import pytest
import torch

from synthetic import to_bf16_bits, bf16_bits_to_f32, weights

HERE = os.path.dirname(os.path.abspath(__file__))
GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _unpack(codes):
    lo = codes & 15
    hi = codes >> 4
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def _grid_value(c):
    c = np.asarray(c)
    return np.where(c & 8, -1.0, 1.0) * GRID[c & 7]


def _e4m3_torch(b):
    return torch.from_numpy(np.asarray(b, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_worked_example(oracle_mod):
    g = json.load(open(os.path.join(HERE, "golden", "nvfp4_worked_example.json")))
    x = np.array(g["x"], np.float32).reshape(1, -1)
    codes, scales, ts = oracle_mod.nvfp4_quantize(x)
    assert ts[0] == np.float32(g["tensor_scale"])
    assert [f"{b:02X}" for b in scales[0]] == g["scales_hex"]
    assert [f"{c:X}" for c in _unpack(codes)[0]] == g["codes_per_element_hex"]
    assert [f"{b:02X}" for b in codes[0]] == g["packed_hex"]


def _grid_tensor(rng, rows, cols, k):
    """A tensor whose quantization is exact: tensor scale 2^k, every block =
    E2M1 grid values (max |g| = 6) times an E4M3 byte's value times 2^k, and one
    block with byte 0x7E so that amax = 6*448*2^k."""
    nb = cols // 16
    g = rng.integers(0, 16, (rows, cols)).astype(np.uint8)
    g = g.reshape(rows, nb, 16)
    g[:, :, 0] = (g[:, :, 0] & 8) | 7                     # max |g| = 6 in each block
    b = rng.integers(0x08, 0x7F, (rows, nb)).astype(np.uint8)  # normal E4M3 bytes
    b[0, 0] = 0x7E
    vals = _grid_value(g) * _e4m3_torch(b)[:, :, None] * 2.0 ** k
    x = vals.reshape(rows, cols).astype(np.float32)
    assert np.array_equal(x.astype(np.float64), vals.reshape(rows, cols))
    return x, g.reshape(rows, cols), b


@pytest.mark.parametrize("k", [-20, -3, 0, 5])
def test_exact_roundtrip_of_grid_tensor(oracle_mod, k):
    rng = np.random.default_rng(100 + k)
    x, g, b = _grid_tensor(rng, 8, 128, k)
    codes, scales, ts = oracle_mod.nvfp4_quantize(x)
    assert ts[0] == np.float32(2.0 ** k)
    assert np.array_equal(scales, b)
    # +-0 codes: value 0 keeps its sign bit
    assert np.array_equal(_unpack(codes), g)
    y = oracle_mod.nvfp4_dequantize(codes, scales, ts)
    assert np.array_equal(y, x)


def test_power_of_two_equivariance(oracle_mod):
    x = weights(16, 256, 1.0, 0.01, 10.0, seed=3)
    c0, s0, t0 = oracle_mod.nvfp4_quantize(x)
    for j in (-7, -1, 1, 9):
        c, s, t = oracle_mod.nvfp4_quantize((x * np.float32(2.0 ** j)).astype(np.float32))
        assert np.array_equal(c, c0) and np.array_equal(s, s0)
        assert t[0] == np.float32(t0[0] * 2.0 ** j)


def test_sign_symmetry(oracle_mod):
    x = weights(16, 256, 1.0, 0.01, 10.0, seed=4)
    c0, s0, t0 = oracle_mod.nvfp4_quantize(x)
    c1, s1, t1 = oracle_mod.nvfp4_quantize(-x)
    assert np.array_equal(s0, s1) and t0[0] == t1[0]
    assert np.array_equal(c1, c0 ^ 0x88)


def test_permutation_within_block(oracle_mod):
    rng = np.random.default_rng(5)
    x = weights(4, 64, 1.0, 0.0, 1.0, seed=5)
    perm = rng.permutation(16)
    xp = x.reshape(4, 4, 16)[:, :, perm].reshape(4, 64)
    c0, s0, _ = oracle_mod.nvfp4_quantize(x)
    c1, s1, _ = oracle_mod.nvfp4_quantize(xp)
    assert np.array_equal(s0, s1)
    u0 = _unpack(c0).reshape(4, 4, 16)[:, :, perm].reshape(4, 64)
    assert np.array_equal(_unpack(c1), u0)


def test_amax_block(oracle_mod):
    x = weights(32, 512, 1.0, 0.01, 10.0, seed=6)
    codes, scales, ts = oracle_mod.nvfp4_quantize(x)
    r, c = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert scales[r, c // 16] == 0x7E
    code = _unpack(codes)[r, c]
    assert code & 7 == 7 and bool(code & 8) == bool(x[r, c] < 0)
    assert ts[0] == np.float32(np.abs(x).max() / np.float32(2688.0))


def test_error_bound(oracle_mod):
    x = weights(64, 1024, 0.02, 0.001, 20.0, seed=7)
    codes, scales, ts = oracle_mod.nvfp4_quantize(x)
    y = oracle_mod.nvfp4_dequantize(codes, scales, ts).astype(np.float64)
    d = (_e4m3_torch(scales) * np.float64(ts[0])).repeat(16, axis=1)
    q = np.abs(x.astype(np.float64)) / d
    # half the local grid step of |x|/d, or the overshoot beyond 6 (saturation)
    step = np.where(q < 2, 0.5, np.where(q < 4, 1.0, 2.0))
    bound = np.maximum(step / 2, q - 6.0) * d
    err = np.abs(x - y)
    assert np.all(err <= bound * (1 + 1e-6) + 1e-30)
    # normal E4M3 scales keep |x|/d at most 6*16/15 (one E4M3 half-ulp below)
    normal = scales >= 0x08
    assert np.all(q.reshape(64, -1, 16).max(axis=2)[normal] <= 6.4 * (1 + 1e-6))


def test_storage_identity(oracle_mod):
    rows, cols = 64, 512
    codes, scales, ts = oracle_mod.nvfp4_quantize(weights(rows, cols, seed=8))
    nbits = 8 * (codes.nbytes + scales.nbytes) + 32 * ts.size
    # 4 bits per element + 8 bits per 16 = 4.5 bits/value, plus one fp32 per tensor
    assert nbits == 4.5 * rows * cols + 32
    # "about 3.5x smaller than FP16, about 1.8x smaller than FP8" ("NVFP4", Technical principle)
    assert round(16 / 4.5, 2) == 3.56 and round(8 / 4.5, 2) == 1.78


def test_dequantize_is_rounded_exact_product(oracle_mod):
    x = weights(32, 256, 0.02, 0.01, 20.0, seed=9)
    codes, scales, ts = oracle_mod.nvfp4_quantize(x)
    exact = (_grid_value(_unpack(codes)) * _e4m3_torch(scales).repeat(16, axis=1)
             * np.float64(ts[0]))
    y = oracle_mod.nvfp4_dequantize(codes, scales, ts)
    assert np.array_equal(y, exact.astype(np.float32))          # one RNE rounding
    assert np.array_equal(oracle_mod.nvfp4_to_f64(codes, scales, ts), exact)


def test_per_row_equals_rowwise_tensors(oracle_mod):
    x = weights(12, 160, 1.0, 0.05, 30.0, seed=11)
    c, s, t = oracle_mod.nvfp4_quantize(x, per_row=True)
    assert t.shape == (12,)
    for r in range(12):
        cr, sr, tr = oracle_mod.nvfp4_quantize(x[r:r + 1])
        assert np.array_equal(c[r], cr[0]) and np.array_equal(s[r], sr[0]) and t[r] == tr[0]


def test_bf16_input_is_widened_exactly(oracle_mod):
    xf = weights(8, 256, 1.0, 0.01, 10.0, seed=12)
    xb = to_bf16_bits(xf)
    a = oracle_mod.nvfp4_quantize(xb)
    b = oracle_mod.nvfp4_quantize(bf16_bits_to_f32(xb))
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_zero_tensor_and_zero_block(oracle_mod):
    x = np.zeros((2, 32), np.float32)
    x[1, 3] = -0.0
    c, s, t = oracle_mod.nvfp4_quantize(x)
    assert t[0] == 0.0 and np.all(s == 0)
    u = _unpack(c)
    assert u[1, 3] == 8 and np.all(np.delete(u.ravel(), 32 + 3) == 0)
    # a zero block inside a non-zero tensor
    x = weights(1, 32, seed=13)
    x[0, 16:] = 0.0
    c, s, t = oracle_mod.nvfp4_quantize(x)
    assert s[0, 1] == 0 and np.all(_unpack(c)[0, 16:] == 0)


def test_rejects_partial_blocks(oracle_mod):
    with pytest.raises(ValueError):
        oracle_mod.nvfp4_quantize(np.zeros((2, 24), np.float32))
