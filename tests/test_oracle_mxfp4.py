"""Pins for the oracle's MXFP4 quantize / dequantize (CPU only).

MXFP4 as the edge-FP4 article (eefocus.com), section "FP4 as the next core
standard", describes it: OCP MX block floating point, 32 contiguous elements
sharing one E8M0 scale, E2M1 elements, 4.25 bits per weight.  Pins: a
hand-worked example for both scale rules, exact round trips, power-of-two
equivariance, the saturation case, the storage identity, and the "NVFP4" page's
claim (section "Technical principle") that 16-blocks track local range better
than MXFP4's 32-blocks.
"""
import json
import os

import numpy as np
import pytest
import torch

from synthetic import weights, to_bf16_bits

HERE = os.path.dirname(os.path.abspath(__file__))
GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _unpack(codes):
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = codes & 15
    out[..., 1::2] = codes >> 4
    return out


def _grid_value(c):
    c = np.asarray(c)
    return np.where(c & 8, -1.0, 1.0) * GRID[c & 7]


@pytest.mark.parametrize("rule,key", [(0, "ocp"), (1, "ceil")])
def test_worked_example(oracle_mod, rule, key):
    g = json.load(open(os.path.join(HERE, "golden", "mxfp4_worked_example.json")))
    x = np.array(g["x"], np.float32).reshape(1, -1)
    codes, scales = oracle_mod.mxfp4_quantize(x, rule)
    assert [f"{b:02X}" for b in scales[0]] == g[key]["scales_hex"]
    u = _unpack(codes)[0].reshape(3, 32)
    for blk in range(3):
        assert [f"{c:X}" for c in u[blk, :10]] == g[key]["codes_first10_per_block_hex"][blk]


@pytest.mark.parametrize("rule", [0, 1])
@pytest.mark.parametrize("top", [4, 6])
def test_exact_roundtrip(oracle_mod, rule, top):
    rng = np.random.default_rng(top + 10 * rule)
    rows, cols = 8, 256
    g = rng.integers(0, 16, (rows, cols // 32, 32)).astype(np.uint8)
    g[..., 0] = (g[..., 0] & 8) | (6 if top == 4 else 7)
    g[..., 1:] = np.where((g[..., 1:] & 7) > (6 if top == 4 else 7), g[..., 1:] & 8, g[..., 1:])
    k = rng.integers(-100, 100, (rows, cols // 32))
    x = (_grid_value(g) * np.exp2(k)[..., None]).reshape(rows, cols).astype(np.float32)
    codes, scales = oracle_mod.mxfp4_quantize(x, rule)
    assert np.array_equal(scales.astype(int), k + 127)
    assert np.array_equal(_unpack(codes), g.reshape(rows, cols))
    assert np.array_equal(oracle_mod.mxfp4_dequantize(codes, scales), x)


@pytest.mark.parametrize("rule", [0, 1])
def test_power_of_two_equivariance(oracle_mod, rule):
    x = weights(8, 256, 1.0, 0.01, 10.0, seed=21)
    c0, s0 = oracle_mod.mxfp4_quantize(x, rule)
    for j in (-5, 3):
        c, s = oracle_mod.mxfp4_quantize((x * np.float32(2.0 ** j)).astype(np.float32), rule)
        assert np.array_equal(c, c0)
        assert np.array_equal(s.astype(int), s0.astype(int) + j)


def test_ocp_rule_saturates_ceil_rule_does_not(oracle_mod):
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 7.5          # floor(log2 7.5) = 2 -> OCP k = 0 -> 7.5 clips to 6
    x[0, 1] = -7.0
    c, s = oracle_mod.mxfp4_quantize(x, 0)
    assert s[0, 0] == 127 and _unpack(c)[0, 0] == 0x7 and _unpack(c)[0, 1] == 0xF
    c, s = oracle_mod.mxfp4_quantize(x, 1)
    assert s[0, 0] == 128                    # 6 * 2^1 = 12 >= 7.5
    assert _unpack(c)[0, 0] == 0x6 and _unpack(c)[0, 1] == 0xE   # 3.75 -> 4, -3.5 -> -4


def test_scale_clamps_to_e8m0_range(oracle_mod):
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = np.float32(2.0 ** -140)        # floor(log2) - 2 = -142 -> clamp to -127
    c, s = oracle_mod.mxfp4_quantize(x, 0)
    assert s[0, 0] == 0
    # 2^-140 * 2^127 = 2^-13 rounds to 0
    assert _unpack(c)[0, 0] == 0


def test_storage_identity(oracle_mod):
    rows, cols = 16, 512
    codes, scales = oracle_mod.mxfp4_quantize(weights(rows, cols, seed=22))
    assert 8 * (codes.nbytes + scales.nbytes) == 4.25 * rows * cols


def test_dequant_is_exact_product(oracle_mod):
    x = weights(8, 256, 0.02, 0.01, 20.0, seed=23)
    codes, scales = oracle_mod.mxfp4_quantize(x)
    e8 = torch.from_numpy(scales).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    exact = _grid_value(_unpack(codes)) * e8.repeat(32, axis=1)
    assert np.array_equal(oracle_mod.mxfp4_to_f64(codes, scales), exact)
    assert np.array_equal(oracle_mod.mxfp4_dequantize(codes, scales), exact.astype(np.float32))


def test_nvfp4_error_below_mxfp4(oracle_mod):
    # heavy-tailed weights and activation-like data, same bf16 inputs for both
    for x in (weights(256, 1024, 0.02, 0.001, 20.0, seed=24),
              weights(256, 1024, 1.0, 0.01, 10.0, seed=25)):
        xb = to_bf16_bits(x)
        xf = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        nv = oracle_mod.nvfp4_to_f64(*oracle_mod.nvfp4_quantize(xb))
        mx = oracle_mod.mxfp4_to_f64(*oracle_mod.mxfp4_quantize(xb))
        e_nv = np.linalg.norm(nv - xf) / np.linalg.norm(xf)
        e_mx = np.linalg.norm(mx - xf) / np.linalg.norm(xf)
        assert e_nv < e_mx
