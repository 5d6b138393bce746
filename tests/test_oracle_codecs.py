"""Pins for the oracle's element and scale codecs (CPU only).

Each codec is checked against something other than itself: the E2M1 grid the
"NVFP4" page (section "Technical principle") and the workload statement fix, an
independent nearest-grid-point search, and torch's own float8_e4m3fn /
float8_e8m0fnu / bfloat16 casts (library codecs written by others).
"""
import os

import numpy as np
import pytest
import torch

HERE = os.path.dirname(os.path.abspath(__file__))


def _grid():
    g = {}
    with open(os.path.join(HERE, "golden", "e2m1_grid.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                c, v = line.split()
                g[int(c)] = float(v)
    return np.array([g[i] for i in range(8)])


GRID = _grid()


def test_e2m1_decode_all_codes(oracle_mod):
    for c in range(16):
        v = oracle_mod.e2m1_decode(c)
        mag = GRID[c & 7]
        assert abs(v) == mag
        assert np.signbit(v) == bool(c & 8)
    # range about +-6 ("NVFP4", Technical principle)
    assert oracle_mod.e2m1_decode(7) == 6.0 and oracle_mod.e2m1_decode(15) == -6.0


def _argmin_e2m1(v: np.ndarray) -> np.ndarray:
    """Independent definition: nearest grid magnitude; a tie goes to the code
    whose mantissa bit (bit 0) is 0; beyond 6 the nearest point is 6 anyway."""
    # every magnitude above 8 has 6 as its nearest grid point; clipping there
    # keeps the fp64 distances exact for huge inputs
    a = np.minimum(np.abs(v.astype(np.float64)), 8.0)
    d = np.abs(a[:, None] - GRID[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among tied candidates prefer even code index
    even = cand & (np.arange(8)[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    return (pick | (np.signbit(v) * 8)).astype(np.uint8)


def _near(values, ulps=96):
    out = []
    for t in values:
        t32 = np.float32(t)
        up = down = t32
        for _ in range(ulps):
            up = np.nextafter(up, np.float32(np.inf))
            down = np.nextafter(down, np.float32(0))
            out += [up, down]
        out.append(t32)
    return np.array(out, np.float32)


def test_e2m1_encode_vs_argmin(oracle_mod):
    # every bfloat16 bit pattern that is finite, as fp32
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    allbf = bits.view(np.float32)
    allbf = allbf[np.isfinite(allbf)]
    # fp32 neighbourhoods of every grid point and every midpoint
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    near = _near(list(GRID) + mids)
    near = np.concatenate([near, -near])
    rng = np.random.default_rng(123)
    rnd = (rng.standard_normal(1_000_000) * np.exp2(rng.integers(-8, 8, 1_000_000))).astype(np.float32)
    v = np.concatenate([allbf, near, rnd])
    got = oracle_mod.e2m1_encode_array(v)
    want = _argmin_e2m1(v)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (v[bad[:5]], got[bad[:5]], want[bad[:5]])


@pytest.mark.parametrize("v,code", [
    (0.25, 0x0), (0.75, 0x2), (1.25, 0x2), (1.75, 0x4), (2.5, 0x4), (3.5, 0x6), (5.0, 0x6),
    (-0.25, 0x8), (-0.75, 0xA), (-5.0, 0xE), (6.0, 0x7), (7.0, 0x7), (1e30, 0x7),
    (float("inf"), 0x7), (-0.0, 0x8), (0.0, 0x0), (-1e-40, 0x8)])
def test_e2m1_ties_saturation_and_signed_zero(oracle_mod, v, code):
    assert oracle_mod.e2m1_encode(v) == code


def test_e2m1_monotone(oracle_mod):
    v = np.linspace(0, 8, 100001, dtype=np.float32)
    c = oracle_mod.e2m1_encode_array(v)
    mags = GRID[c & 7]
    assert np.all(np.diff(mags) >= 0)


def test_e2m1_roundtrip(oracle_mod):
    for c in range(16):
        assert oracle_mod.e2m1_encode(oracle_mod.e2m1_decode(c)) == c


# ----------------------------------------------------------------- E4M3 --

def _torch_e4m3_decode(b: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(b.astype(np.uint8)).view(torch.float8_e4m3fn).to(torch.float64)
    return t.numpy()


def test_e4m3_decode_all_bytes_vs_torch(oracle_mod):
    b = np.arange(256, dtype=np.uint8)
    ref = _torch_e4m3_decode(b)
    got = np.array([oracle_mod.e4m3_decode(int(x)) for x in b])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert np.array_equal(got[~nan], ref[~nan])
    assert oracle_mod.e4m3_decode(0x7E) == 448.0
    assert oracle_mod.e4m3_decode(0x01) == 2.0 ** -9
    assert oracle_mod.e4m3_decode(0x08) == 2.0 ** -6


def test_e4m3_encode_vs_torch_cast(oracle_mod):
    # torch's fp32 -> float8_e4m3fn cast rounds to nearest even; it agrees with a
    # saturating encoder for every value up to the 448|480 midpoint (464).
    bits = np.arange(1 << 15, dtype=np.uint32) << 16      # non-negative bf16 patterns
    v = bits.view(np.float32)
    vals = [oracle_mod.e4m3_decode(b) for b in range(0x7F)]
    mids = [(vals[i] + vals[i + 1]) / 2 for i in range(0x7E)]
    near = _near(vals + mids, ulps=48)
    rng = np.random.default_rng(7)
    rnd = (rng.random(2_000_000) * np.exp2(rng.integers(-12, 9, 2_000_000))).astype(np.float32)
    v = np.concatenate([v, near, rnd])
    v = v[np.isfinite(v) & (v >= 0) & (v <= 464.0)]
    got = oracle_mod.e4m3_encode_array(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (v[bad[:5]], got[bad[:5]], ref[bad[:5]])


@pytest.mark.parametrize("q", [448.0, 464.0, 464.0001, 480.0, 1e6, 3.0e38, float("inf")])
def test_e4m3_encode_saturates(oracle_mod, q):
    assert oracle_mod.e4m3_encode_sat(q) == 0x7E


def test_e4m3_encode_roundtrip_nonnegative(oracle_mod):
    for b in range(0x7F):
        assert oracle_mod.e4m3_encode_sat(oracle_mod.e4m3_decode(b)) == b


def test_e4m3_subnormal_ties(oracle_mod):
    assert oracle_mod.e4m3_encode_sat(2.0 ** -10) == 0x00      # 0.5 ulp -> even 0
    assert oracle_mod.e4m3_encode_sat(3 * 2.0 ** -10) == 0x02  # 1.5 -> 2
    assert oracle_mod.e4m3_encode_sat(2.0 ** -6 * 0.999) == 0x08


# ----------------------------------------------------------------- E8M0 --

def test_e8m0_all_bytes_vs_torch(oracle_mod):
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = np.array([oracle_mod.e8m0_decode(int(x)) for x in b])
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])
    assert got[127] == 1.0


# ----------------------------------------------------------------- bf16 --

def test_bf16_rne_vs_torch(oracle_mod):
    rng = np.random.default_rng(5)
    v = rng.standard_normal(1_000_000).astype(np.float32) * np.float32(1000)
    ties = (np.arange(1 << 16, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    ties = ties[np.isfinite(ties)]
    v = np.concatenate([v, ties, np.array([0.0, -0.0, 1e-40, -1e-40], np.float32)])
    got = oracle_mod.f32_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
