"""GPU parity: NVFP4 / MXFP4 quantize and dequantize, bit-exact against the oracle.

Codes, scale bytes and tensor scales are integers / exact floats: the HIP path
must reproduce the oracle's bytes exactly, on the workloads at full size, on
ragged shapes, and on adversarial values (midpoint ties, +-1 ulp around them,
subnormals, zero blocks, signed zeros, tiny and huge tensors).
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import (assert_bytes_equal, bf16bits_to_dev, bf16_tensor_bits, dev, f32_to_dev, log)
from synthetic import WORKLOADS, activations_f32, bf16_bits_to_f32, to_bf16_bits, weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import block_scaled_fp4_04_amd as fp4

    assert fp4.lib().fp4blk_check_device() == 0, "current device is not a gfx950"


def fp4():
    import block_scaled_fp4_04_amd as m

    return m


def _nv_check(x_np, mode="tensor", what=""):
    """Quantize x (fp32 array or bf16 bits) on the GPU and compare with the oracle."""
    per_row = mode == "row"
    log(f"nvfp4_quantize {what} shape={x_np.shape} dtype={x_np.dtype} mode={mode}")
    xt = f32_to_dev(x_np) if x_np.dtype == np.float32 else bf16bits_to_dev(x_np)
    p = fp4().nvfp4_quantize(xt, mode=mode)
    torch.cuda.synchronize()
    oc, os_, ot = oracle.nvfp4_quantize(x_np, per_row=per_row)
    assert_bytes_equal(p.scales, os_, f"scales {what}")
    assert_bytes_equal(p.codes, oc, f"codes {what}")
    assert np.array_equal(p.tscale.cpu().numpy().view(np.uint32), ot.view(np.uint32)), f"tscale {what}"
    return p, (oc, os_, ot)


# ----------------------------------------------------------- workloads ----

def test_tiny_workload_roundtrip():
    wl = WORKLOADS["tiny_roundtrip_256"]
    w = wl.weights()
    p, (oc, os_, ot) = _nv_check(w, "tensor", "tiny 256x256")
    y = fp4().nvfp4_dequantize(p)
    torch.cuda.synchronize()
    yo = oracle.nvfp4_dequantize(oc, os_, ot)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), yo.view(np.uint32))


def test_decode_weights_full_size():
    wl = WORKLOADS["decode_gemv_k5120_n17408"]
    _nv_check(wl.weights(), "tensor", "decode weights 17408x5120")


def test_prefill_activations_per_row_full_size():
    wl = WORKLOADS["prefill_w4a4_m4096"]
    _nv_check(wl.activations_bf16(4096), "row", "prefill activations 4096x5120 bf16")


# ------------------------------------------------------------ ragged ------

@pytest.mark.parametrize("rows,cols", [(1, 16), (3, 48), (17, 80), (33, 1040), (130, 5120), (257, 272),
                                       (5, 8192), (3, 8208), (2, 16384)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["tensor", "row"])
def test_ragged_shapes(rows, cols, dtype, mode):
    x = weights(rows, cols, 1.0, 0.02, 25.0, seed=rows * 1000 + cols)
    if dtype == "bf16":
        x = to_bf16_bits(x)
    _nv_check(x, mode, f"ragged {rows}x{cols}")


@pytest.mark.parametrize("mode", ["tensor", "row"])
def test_strided_input(mode):
    x = weights(40, 160, 1.0, 0.01, 10.0, seed=77)
    big = torch.zeros(40, 256, dtype=torch.float32, device=dev())
    big[:, :160] = f32_to_dev(x)
    view = big[:, :160]
    p = fp4().nvfp4_quantize(view, mode=mode)
    torch.cuda.synchronize()
    oc, os_, ot = oracle.nvfp4_quantize(x, per_row=mode == "row")
    assert_bytes_equal(p.codes, oc, "strided codes")
    assert_bytes_equal(p.scales, os_, "strided scales")
    assert np.array_equal(p.tscale.cpu().numpy(), ot), "strided tensor scale(s)"


# ------------------------------------------------------- adversarial ------

def _midpoint_tensor(seed):
    """Tensor scale 2^-3 (amax 2688 * 2^-3); block scales from E4M3 bytes; the
    elements sit exactly on E2M1 midpoints / grid points times the block divisor,
    and one fp32 ulp either side of them."""
    rng = np.random.default_rng(seed)
    k = -3
    rows, nb = 64, 20
    b = rng.integers(1, 0x7E, (rows, nb)).astype(np.uint8)
    b[0, 0] = 0x7E
    d = np.array([[oracle.e4m3_decode(int(v)) for v in r] for r in b]) * 2.0 ** k
    pts = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, 0.0, 5.5])
    x = np.empty((rows, nb, 16), np.float32)
    for r in range(rows):
        for j in range(nb):
            t = rng.permutation(pts)
            v = (t * d[r, j]).astype(np.float32)
            nudge = rng.integers(-1, 2, 16)
            v = np.where(nudge > 0, np.nextafter(v, np.float32(np.inf)), v)
            v = np.where(nudge < 0, np.nextafter(v, np.float32(0)), v)
            v = np.minimum(v, np.float32(6 * d[r, j]))        # block amax stays 6 * d
            v *= np.where(rng.random(16) < 0.5, -1, 1).astype(np.float32)
            # keep one exact 6*d so this block's scale is b
            v[0] = np.float32(6 * d[r, j])
            x[r, j] = v
    x[0, 0, 0] = np.float32(2688 * 2.0 ** k)
    return x.reshape(rows, nb * 16)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_midpoints_and_neighbours(seed):
    x = _midpoint_tensor(seed)
    _nv_check(x, "tensor", f"midpoints seed {seed}")


def _midpoint_full_scale(seed, per_row):
    """fp32 tensor whose tensor (or row) scale has a full 24-bit mantissa, so the
    block steps d = fl32(E4M3(b) s) do too; elements sit on t d rounded to fp32 and
    up to two ulps either side, t an E2M1 grid point or midpoint, so each code is
    decided by the last bit of the correctly rounded quotient fl32(x / d)."""
    rng = np.random.default_rng(seed)
    rows, nb = 48, 24
    thr = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], np.float32)
    n_s = rows if per_row else 1
    amax = ((1 + rng.random(n_s)) * 2.0 ** rng.integers(-12, 13, n_s)).astype(np.float32)
    s = (amax / np.float32(2688.0)).astype(np.float32)
    x = np.empty((rows, nb, 16), np.float32)
    for r in range(rows):
        sr = s[r if per_row else 0]
        for j in range(nb):
            b = int(rng.integers(1, 0x77))                      # E4M3 bytes up to 240, subnormals included
            bv = np.float32(oracle.e4m3_decode(b))
            d = np.float32(bv * sr)
            v = (rng.choice(thr, 16) * d).astype(np.float32)
            for _ in range(2):
                step = rng.integers(-1, 2, 16)
                v = np.where(step > 0, np.nextafter(v, np.float32(np.inf)), v)
                v = np.where(step < 0, np.nextafter(v, np.float32(0)), v)
            v[0] = np.float32(bv * np.float32(6.0 * sr))        # the block maximum picks byte b
            v *= np.where(rng.random(16) < 0.5, -1, 1).astype(np.float32)
            x[r, j] = rng.permutation(v)
        x[r if per_row else 0, 0, 0] = amax[r if per_row else 0]
    return x.reshape(rows, nb * 16)


@pytest.mark.parametrize("seed", [4, 5, 6])
@pytest.mark.parametrize("mode", ["tensor", "row"])
def test_midpoints_full_mantissa_scale(seed, mode):
    x = _midpoint_full_scale(seed, mode == "row")
    _nv_check(x, mode, f"full-mantissa midpoints seed {seed}")
    _nv_check(to_bf16_bits(x), mode, f"full-mantissa midpoints seed {seed} as bf16")


def test_subnormal_zero_and_signed_zero_blocks():
    rng = np.random.default_rng(9)
    x = weights(8, 256, 1.0, 0.0, 1.0, seed=9)
    x[0, :16] = 0.0
    x[1, 16:32] = -0.0
    x[2, 32:48] = (rng.standard_normal(16) * 1e-41).astype(np.float32)   # fp32 subnormals
    x[3, :16] = np.float32(1e-9)                                          # E4M3 underflow -> d = 0
    x[3, 1] = np.float32(-1e-9)
    x[4, :] = np.float32(2.0) ** rng.integers(-20, 5, 256)               # powers of two
    x[5, 7] = np.float32(3.0e4)                                           # single outlier
    _nv_check(x, "tensor", "special blocks")
    _nv_check(x, "row", "special blocks per row")


# the quantizers switch from the shared-reciprocal division to the IEEE division
# when the tensor scale leaves [2^-50, 2^50]: amax 2688 * 2^-50 ~ 2.39e-12 and
# 2688 * 2^50 ~ 3.03e18; both sides of each edge are covered
@pytest.mark.parametrize("scale", [1e-38, 1e-30, 2.0e-13, 2.2e-13, 2.6e-13, 3e-12, 2.7e17, 3.1e17, 1e30, 3e36])
@pytest.mark.parametrize("mode", ["tensor", "row"])
def test_tiny_and_huge_tensors(scale, mode):
    x = (weights(4, 64, 1.0, 0.05, 10.0, seed=5) * np.float32(scale)).astype(np.float32)
    _nv_check(x, mode, f"scaled by {scale}")
    if mode == "row":
        _nv_check(to_bf16_bits(x), mode, f"scaled by {scale}, bf16")


@pytest.mark.parametrize("edge", [-50, 50])
@pytest.mark.parametrize("mode", ["tensor", "row"])
def test_scale_at_fast_path_edges(edge, mode):
    """Rows whose amax puts s = amax / 2688 one ulp inside, on and one ulp outside 2^edge."""
    rows = []
    for k, base in enumerate(weights(9, 128, 1.0, 0.05, 10.0, seed=21)):
        target = np.float32(2.0 ** edge * 2688.0)
        amax = [np.nextafter(target, np.float32(0)), target, np.nextafter(target, np.float32(np.inf))][k % 3]
        r = (base / np.abs(base).max() * amax).astype(np.float32)
        r[np.argmax(np.abs(r))] = amax
        rows.append(r)
    x = np.stack(rows)
    if mode == "tensor":
        for r in x:
            _nv_check(r[None, :], mode, f"edge 2^{edge}")
    else:
        _nv_check(x, mode, f"edge 2^{edge}")


def test_all_zero_tensor():
    _nv_check(np.zeros((3, 32), np.float32), "tensor", "all zero")


def test_nonfinite_flag():
    x = weights(8, 64, seed=3)
    x[2, 5] = np.inf
    flag = torch.zeros(1, dtype=torch.int32, device=dev())
    fp4().nvfp4_quantize(f32_to_dev(x), nonfinite=flag)
    torch.cuda.synchronize()
    assert flag.item() == 1
    flag.zero_()
    fp4().nvfp4_quantize(f32_to_dev(weights(8, 64, seed=4)), nonfinite=flag)
    fp4().nvfp4_quantize(bf16bits_to_dev(to_bf16_bits(weights(8, 64, seed=4))), mode="row", nonfinite=flag)
    torch.cuda.synchronize()
    assert flag.item() == 0
    x[2, 5] = np.nan
    fp4().nvfp4_quantize(f32_to_dev(x), mode="row", nonfinite=flag)
    torch.cuda.synchronize()
    assert flag.item() == 1
    flag.zero_()
    fp4().mxfp4_quantize(f32_to_dev(x), nonfinite=flag)
    torch.cuda.synchronize()
    assert flag.item() == 1


def test_deterministic():
    x = f32_to_dev(weights(300, 1024, 0.02, 0.001, 20.0, seed=8))
    a = fp4().nvfp4_quantize(x)
    b = fp4().nvfp4_quantize(x)
    torch.cuda.synchronize()
    assert torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales) and torch.equal(a.tscale, b.tscale)


# --------------------------------------------------------- dequantize -----

@pytest.mark.parametrize("mode", ["tensor", "row"])
def test_dequantize_fp32_and_bf16(mode):
    x = weights(70, 480, 0.02, 0.01, 20.0, seed=12)
    p, (oc, os_, ot) = _nv_check(x, mode, "for dequant")
    y32 = fp4().nvfp4_dequantize(p, torch.float32)
    y16 = fp4().nvfp4_dequantize(p, torch.bfloat16)
    torch.cuda.synchronize()
    yo = oracle.nvfp4_dequantize(oc, os_, ot, per_row=(mode == "row"))
    assert np.array_equal(y32.cpu().numpy().view(np.uint32), yo.view(np.uint32))
    assert np.array_equal(bf16_tensor_bits(y16), oracle.f32_to_bf16_bits(yo))


def test_dequantize_full_decode_weights():
    wl = WORKLOADS["decode_gemv_k5120_n17408"]
    w = wl.weights()
    oc, os_, ot = oracle.nvfp4_quantize(w)
    p = fp4().PackedNVFP4(torch.from_numpy(oc).to(dev()), torch.from_numpy(os_).to(dev()),
                          torch.from_numpy(ot).to(dev()), w.shape[0], w.shape[1])
    log("nvfp4_dequantize decode weights 17408x5120 -> bf16")
    y = fp4().nvfp4_dequantize(p, torch.bfloat16)
    torch.cuda.synchronize()
    yo = oracle.nvfp4_dequantize(oc, os_, ot)
    assert np.array_equal(bf16_tensor_bits(y), oracle.f32_to_bf16_bits(yo))


# -------------------------------------------------------------- MXFP4 -----

def _mx_check(x_np, rule, what):
    log(f"mxfp4_quantize {what} shape={x_np.shape} dtype={x_np.dtype} rule={rule}")
    xt = f32_to_dev(x_np) if x_np.dtype == np.float32 else bf16bits_to_dev(x_np)
    p = fp4().mxfp4_quantize(xt, rule=rule)
    torch.cuda.synchronize()
    oc, os_ = oracle.mxfp4_quantize(x_np, oracle.MX_OCP_FLOOR if rule == "ocp" else oracle.MX_CEIL)
    assert_bytes_equal(p.scales, os_, f"mx scales {what}")
    assert_bytes_equal(p.codes, oc, f"mx codes {what}")
    return p, (oc, os_)


@pytest.mark.parametrize("rule", ["ocp", "ceil"])
@pytest.mark.parametrize("rows,cols", [(1, 32), (5, 96), (33, 1056), (130, 5120)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mxfp4_ragged(rule, rows, cols, dtype):
    x = weights(rows, cols, 1.0, 0.02, 25.0, seed=rows + cols)
    if dtype == "bf16":
        x = to_bf16_bits(x)
    _mx_check(x, rule, f"ragged {rows}x{cols}")


@pytest.mark.parametrize("rule", ["ocp", "ceil"])
def test_mxfp4_adversarial(rule):
    rng = np.random.default_rng(4)
    x = weights(16, 256, 1.0, 0.0, 1.0, seed=4)
    x[0, :32] = 0.0
    x[1, :32] = -0.0
    x[2, :32] = (rng.standard_normal(32) * 1e-42).astype(np.float32)      # subnormal block (k clamps)
    x[3, :32] = np.float32(7.0); x[3, 1] = np.float32(-7.5)                 # OCP saturation
    x[4, :32] = np.float32(6.0) * np.float32(2.0) ** rng.integers(-3, 3, 32)
    x[5, :32] = np.float32(1.5); x[5, 0] = np.float32(6.0)                  # ceil boundary 1.5*2^E
    x[6, :32] = np.float32(3e38)                                            # huge
    x[7, :] = np.float32(2.0) ** rng.integers(-140, 120, 256)
    # grid midpoints times the block's power of two
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 4, np.float32)
    x[8, :32] = rng.permutation(mids) * np.float32(0.125)
    _mx_check(x, rule, "adversarial")


def test_mxfp4_dequantize():
    x = weights(40, 320, 0.02, 0.01, 20.0, seed=13)
    p, (oc, os_) = _mx_check(x, "ocp", "for dequant")
    y32 = fp4().mxfp4_dequantize(p, torch.float32)
    y16 = fp4().mxfp4_dequantize(p, torch.bfloat16)
    torch.cuda.synchronize()
    yo = oracle.mxfp4_dequantize(oc, os_)
    assert np.array_equal(y32.cpu().numpy().view(np.uint32), yo.view(np.uint32))
    assert np.array_equal(bf16_tensor_bits(y16), oracle.f32_to_bf16_bits(yo))


def test_mxfp4_dequantize_every_scale_and_code():
    """Every E8M0 byte (0..254 and the NaN byte 0xFF) with all 16 codes in both
    nibble positions: fp32 and bf16 bits equal the oracle's (subnormal results at
    the low end, overflow to infinity at the high end, NaN for 0xFF)."""
    rows, cols = 256, 64
    codes = np.empty((rows, cols // 2), np.uint8)
    lo = np.arange(32, dtype=np.uint8) % 16
    hi = (np.arange(32, dtype=np.uint8) * 7 + 3) % 16
    codes[:] = lo | (hi << 4)
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], cols // 32, axis=1)
    p = fp4().PackedMXFP4(torch.from_numpy(codes).to(dev()), torch.from_numpy(scales).to(dev()), rows, cols)
    y32 = fp4().mxfp4_dequantize(p, torch.float32)
    y16 = fp4().mxfp4_dequantize(p, torch.bfloat16)
    torch.cuda.synchronize()
    yo = oracle.mxfp4_dequantize(codes, scales)
    assert np.isnan(yo[255]).all() and np.isinf(yo[254]).any() and (yo[0] != 0).any()
    got = y32.cpu().numpy().view(np.uint32)
    bad = np.argwhere(got != yo.view(np.uint32))
    assert bad.size == 0, f"{len(bad)} fp32 mismatches, first (row = scale byte, col) {bad[:4].tolist()}"
    assert np.array_equal(bf16_tensor_bits(y16), oracle.f32_to_bf16_bits(yo))


def test_mxfp4_full_size_activations():
    wl = WORKLOADS["mx_vs_nv_w4a4_m8192"]
    _mx_check(wl.activations_bf16(8192), "ocp", "activations 8192x5120 bf16")


def test_bf16_equals_widened_fp32():
    xb = to_bf16_bits(activations_f32(64, 512, 0.01, 30.0, seed=2))
    pb, _ = _nv_check(xb, "row", "bf16 rows")
    pf, _ = _nv_check(bf16_bits_to_f32(xb), "row", "widened fp32 rows")
    assert torch.equal(pb.codes, pf.codes) and torch.equal(pb.scales, pf.scales)
