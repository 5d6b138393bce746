"""Pins for the oracle's MXFP8 quantize / dequantize (CPU only): the FP8
activations of W4A8 (edge-FP4 article, eefocus.com: an NPU with native W4A8,
weights quantized to FP4 and activations to FP8).  Reading: OCP MX blocks of 32
elements with an E8M0 scale and E4M3FN elements.

Pins: element codes against torch's float8_e4m3fn cast (a codec written by
others) with the scale exponent recomputed here from the MX definition; exact
round trips of representable blocks under both rules; power-of-two
equivariance; sign symmetry; the saturation case of the OCP rule; the storage
identity (8 + 8/32 bits a value).
"""
import numpy as np
import pytest
import torch

from synthetic import to_bf16_bits, weights


def _k_rule(amax, rule):
    m, e = np.frexp(amax.astype(np.float64))      # amax = m 2^e, m in [0.5, 1)
    E = e - 1                                     # floor(log2 amax)
    if rule == 0:
        k = E - 8
    else:
        k = np.where(amax <= 1.75 * np.exp2(E), E - 8, E - 7)
    return np.clip(k, -127, 127)


def _torch_codes(x, k):
    v = np.clip(np.abs(x.astype(np.float64)) * np.exp2(-k), 0, 448.0)
    mag = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return np.where(np.signbit(x), mag | 0x80, mag).astype(np.uint8)


@pytest.mark.parametrize("rule", [0, 1])
def test_codes_vs_torch_cast(oracle_mod, rule):
    x = weights(64, 256, 1.0, 0.01, 10.0, seed=3 + rule)
    x[5, :32] = 0.0                                  # a zero block
    x[6, 32:64] *= 1e-30                             # tiny block
    codes, scales = oracle_mod.mxfp8_quantize(x, rule)
    blocks = x.reshape(64, 8, 32)
    amax = np.abs(blocks).max(axis=2)
    k = _k_rule(np.where(amax > 0, amax, 1.0), rule)
    want_scales = np.where(amax > 0, k + 127, 0).astype(np.uint8)
    assert np.array_equal(scales, want_scales)
    want = _torch_codes(blocks, np.where(amax > 0, k, 0)[..., None]).reshape(64, 256)
    zero = np.repeat(amax == 0, 32, axis=1)
    want[zero] = np.where(np.signbit(x[zero]), 0x80, 0x00)
    assert np.array_equal(codes, want)


@pytest.mark.parametrize("rule", [0, 1])
def test_roundtrip_of_representable_blocks(oracle_mod, rule):
    rng = np.random.default_rng(5)
    finite = np.array([b for b in range(0x7F)], np.uint8)
    vals = torch.from_numpy(finite).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    rows = []
    for r in range(16):
        k = int(rng.integers(-20, 20))
        blk = rng.choice(vals, 32) * rng.choice([-1.0, 1.0], 32)
        blk[rng.integers(32)] = 448.0                # the block's largest element
        rows.append(blk * 2.0 ** k)
    x = np.array(rows, np.float32).reshape(2, 256)
    codes, scales = oracle_mod.mxfp8_quantize(x, rule)
    back = oracle_mod.mxfp8_to_f64(codes, scales)
    assert np.array_equal(back, x.astype(np.float64))


def test_power_of_two_equivariance_and_sign(oracle_mod):
    x = weights(8, 128, 0.5, 0.01, 10.0, seed=9)
    c0, s0 = oracle_mod.mxfp8_quantize(x)
    c1, s1 = oracle_mod.mxfp8_quantize((x * 2.0 ** 5).astype(np.float32))
    assert np.array_equal(c0, c1) and np.array_equal(s1.astype(int), s0.astype(int) + 5)
    c2, s2 = oracle_mod.mxfp8_quantize(-x)
    assert np.array_equal(c2, c0 ^ 0x80) and np.array_equal(s2, s0)


def test_ocp_rule_saturates_and_ceil_rule_does_not(oracle_mod):
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 1.9 * 2.0 ** 4                         # mantissa 1.9 > 1.75: 448 2^(4-8) = 28 < 30.4
    x[0, 1] = 1.0
    c0, s0 = oracle_mod.mxfp8_quantize(x, 0)
    assert s0[0, 0] == 127 + 4 - 8 and c0[0, 0] == 0x7E
    c1, s1 = oracle_mod.mxfp8_quantize(x, 1)
    assert s1[0, 0] == 127 + 4 - 7
    back = oracle_mod.mxfp8_to_f64(c1, s1)
    assert abs(back[0, 0] - x[0, 0]) <= 2.0 ** (4 - 3) / 2   # within half an E4M3 step at that exponent


def test_storage_identity(oracle_mod):
    x = to_bf16_bits(weights(4, 1024, 1.0, 0.0, 1.0, seed=1))
    codes, scales = oracle_mod.mxfp8_quantize(x)
    assert (codes.nbytes + scales.nbytes) * 8 / x.size == 8.25
