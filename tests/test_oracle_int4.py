"""Pins of the oracle's INT4 baseline quantizer.

INT4 is the integer format FP4 is compared with (edge-FP4 article, eefocus.com,
section on why FP4 suits compression; "NVFP4" wiki, newton.com.tw, competition
section).  The pages fix no layout; the reading is symmetric levels -7..7, one
step d per block, element = round-half-even(x / d) saturated at +-7, with d from
one of four containers.  Pinned here: every code against a brute-force nearest
level (ties to the even level), every step against its container's rule
recomputed with numpy / torch casts, exact round trips, zero blocks.
"""
import numpy as np
import pytest
import torch

import oracle
from synthetic import heavy_tailed


def _brute_codes(x, step, block):
    """Nearest of the 15 levels to x / d, ties to the even level (brute force)."""
    d = np.repeat(step, block, axis=1)
    r = np.divide(x.astype(np.float64), d, out=np.zeros(x.shape), where=d > 0)
    levels = np.arange(-7, 8, dtype=np.float64)
    dist = np.abs(r[..., None] - levels)
    best = dist.min(axis=-1, keepdims=True)
    cand = np.where(dist == best, levels, np.nan)
    even = np.where(np.isnan(cand), np.inf, np.where(cand % 2 == 0, cand, np.inf))
    pick = np.where(np.isinf(even.min(axis=-1)), np.nanmin(cand, axis=-1), even.min(axis=-1))
    return np.where(d > 0, pick, 0).astype(np.int8)


@pytest.mark.parametrize("kind,block", [(oracle.INT4_F32, 64), (oracle.INT4_BF16, 128),
                                        (oracle.INT4_E4M3_TENSOR, 16), (oracle.INT4_E8M0, 32)])
@pytest.mark.parametrize("dist", ["gaussian", "student_t3", "channel_outliers"])
def test_int4_codes_and_steps(kind, block, dist):
    x = heavy_tailed(16, 512, dist, seed=block)
    x[0, :block] = 0.0                                         # a zero block
    codes, step, ts = oracle.int4_quantize(x, block, kind)
    amax_b = np.abs(x).reshape(16, -1, block).max(axis=-1)
    if kind == oracle.INT4_F32:
        want = (amax_b / np.float32(7)).astype(np.float64)
    elif kind == oracle.INT4_BF16:
        want = torch.from_numpy(amax_b / np.float32(7)).to(torch.bfloat16).float().numpy().astype(np.float64)
    elif kind == oracle.INT4_E4M3_TENSOR:
        s = np.float32(np.abs(x).max()) / np.float32(448 * 7)
        assert ts == s
        q = torch.from_numpy(amax_b / (np.float32(7) * s)).to(torch.float8_e4m3fn).float().numpy()
        want = q.astype(np.float64) * np.float64(s)
    else:
        k = np.ceil(np.log2(np.where(amax_b > 0, amax_b, 1) / 7.0))
        want = np.where(amax_b > 0, 2.0 ** k, 0.0)
        nz = amax_b > 0
        assert np.all(7 * want[nz] >= amax_b[nz]) and np.all(3.5 * want[nz] < amax_b[nz])
    want = np.where(amax_b > 0, want, 0.0)
    assert np.array_equal(step, want)
    assert np.array_equal(codes, _brute_codes(x, step, block))
    assert np.all(codes[0, :block] == 0) and step[0, 0] == 0.0


def test_int4_round_trip_of_representable_blocks():
    rng = np.random.default_rng(3)
    q = rng.integers(-7, 8, (8, 128)).astype(np.float32)
    q[:, ::32] = 7.0                                           # amax = 7 d in every block
    d = np.float32(2.0) ** rng.integers(-6, 6, (8, 4)).astype(np.float32)
    x = q * np.repeat(d, 32, axis=1)
    codes, step, _ = oracle.int4_quantize(x, 32, oracle.INT4_E8M0)
    assert np.array_equal(step, d.astype(np.float64)) and np.array_equal(codes, q.astype(np.int8))
    assert np.array_equal(oracle.int4_to_f64(codes, step), x.astype(np.float64))
    codes, step, _ = oracle.int4_quantize(x, 32, oracle.INT4_F32)
    assert np.array_equal(oracle.int4_to_f64(codes, step), x.astype(np.float64))


def test_int4_ties_go_to_the_even_level():
    x = np.array([[7.0, 0.5, 1.5, 2.5, -0.5, -1.5, 3.5, 6.5] * 4], np.float32)   # step 1 (amax 7)
    codes, step, _ = oracle.int4_quantize(x, 32, oracle.INT4_F32)
    assert step[0, 0] == 1.0
    assert codes[0, :8].tolist() == [7, 0, 2, 2, 0, -2, 4, 6]
