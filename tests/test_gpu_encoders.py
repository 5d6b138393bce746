"""GPU parity: the quantizers' E2M1 and E4M3 encoders over every fp32 input that
can reach them, and guard bands around every quantizer and dequantizer output.

The E2M1 element encoder (FP4, "NVFP4" wiki, section "Technical principle":
1 sign, 2 exponent and 1 mantissa bit, range +-6) and the E4M3 encoder (the FP8
block scale of NVFP4 and the MXFP8 elements) are gfx950's scaled conversions.
They are checked here through the public quantizers, with every block given an
anchor value that fixes its E8M0 exponent at k = 0, so every other value of the
block is encoded as itself:

* MXFP4, OCP rule: an anchor of 4 gives floor(log2 amax) - 2 = 0 for blocks
  whose values lie in (-8, 8); the sweep covers every fp32 bit pattern of
  magnitude below 8, both signs (2 x 1,090,519,040 values);
* MXFP8, OCP rule: an anchor of 256 gives floor(log2 amax) - 8 = 0 for values in
  [0, 512); the sweep covers every such fp32 pattern (1,140,850,688 values),
  which includes the saturation range [448, 512).

Each chunk is built twice from the same bit patterns, on the device and on the
host, and the device codes are compared byte for byte with the oracle's.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import dev, log

pytestmark = pytest.mark.gpu

BLOCK_VALUES = 31                 # swept values per 32-block (one slot holds the anchor)
CHUNK_BLOCKS = 1 << 23            # 260,046,848 swept values per chunk
MX4_PATTERNS = 0x41000000         # fp32 bit patterns of 0 .. 8 (exclusive)
MX8_PATTERNS = 0x44000000         # fp32 bit patterns of 0 .. 512 (exclusive)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import block_scaled_fp4_04_amd as fp4

    assert fp4.lib().fp4blk_check_device() == 0, "current device is not a gfx950"


def fp4():
    import block_scaled_fp4_04_amd as m

    return m


def _chunks(total):
    per = CHUNK_BLOCKS * BLOCK_VALUES
    return [(p, min(total, p + per)) for p in range(0, total, per)]


def _sweep_host(p0, p1, anchor, negate):
    n = p1 - p0
    nblk = -(-n // BLOCK_VALUES)
    pat = np.arange(p0, p0 + nblk * BLOCK_VALUES, dtype=np.uint32)
    pat[n:] = 0                                          # pad the last block with zeros
    x = np.empty((nblk, 32), np.float32)
    x[:, 0] = anchor
    x[:, 1:] = pat.view(np.float32).reshape(nblk, BLOCK_VALUES)
    if negate:
        x[:, 1:] = -x[:, 1:]
    return x.reshape(-1, 4096) if nblk % 128 == 0 else x


def _sweep_dev(p0, p1, anchor, negate):
    n = p1 - p0
    nblk = -(-n // BLOCK_VALUES)
    pat = torch.arange(p0, p0 + nblk * BLOCK_VALUES, dtype=torch.int64, device=dev())
    pat[n:] = 0
    x = torch.empty(nblk, 32, dtype=torch.float32, device=dev())
    x[:, 0] = anchor
    x[:, 1:] = pat.to(torch.int32).view(torch.float32).view(nblk, BLOCK_VALUES)
    if negate:
        x[:, 1:] = -x[:, 1:]
    return x.view(-1, 4096) if nblk % 128 == 0 else x


def _compare(got: torch.Tensor, want: np.ndarray, what: str):
    g = got.cpu().numpy()
    assert g.shape == want.shape, (what, g.shape, want.shape)
    bad = np.flatnonzero(g.reshape(-1) != want.reshape(-1))
    assert bad.size == 0, f"{what}: {bad.size} bytes differ, first at flat index {bad[:4].tolist()}"


@pytest.mark.parametrize("negate", [False, True])
@pytest.mark.parametrize("chunk", range(len(_chunks(MX4_PATTERNS))))
def test_e2m1_encoder_every_fp32_below_8(chunk, negate):
    p0, p1 = _chunks(MX4_PATTERNS)[chunk]
    log(f"MXFP4 k=0 sweep, patterns {p0:#x}..{p1:#x}, negated={negate}")
    xd = _sweep_dev(p0, p1, 4.0, negate)
    p = fp4().mxfp4_quantize(xd, rule="ocp")
    torch.cuda.synchronize()
    del xd
    xh = _sweep_host(p0, p1, 4.0, negate)
    oc, os_ = oracle.mxfp4_quantize(xh, oracle.MX_OCP_FLOOR)
    assert np.all(os_ == 127), "every sweep block should have E8M0 byte 127 (k = 0)"
    _compare(p.scales, os_, "E8M0 bytes")
    _compare(p.codes, oc, "E2M1 codes")


@pytest.mark.parametrize("chunk", range(len(_chunks(MX8_PATTERNS))))
def test_e4m3_encoder_every_fp32_below_512(chunk):
    p0, p1 = _chunks(MX8_PATTERNS)[chunk]
    log(f"MXFP8 k=0 sweep, patterns {p0:#x}..{p1:#x}")
    xd = _sweep_dev(p0, p1, 256.0, False)
    p = fp4().mxfp8_quantize(xd, rule="ocp")
    torch.cuda.synchronize()
    del xd
    xh = _sweep_host(p0, p1, 256.0, False)
    oc, os_ = oracle.mxfp8_quantize(xh, oracle.MX_OCP_FLOOR)
    assert np.all(os_ == 127), "every sweep block should have E8M0 byte 127 (k = 0)"
    _compare(p.scales, os_, "E8M0 bytes")
    _compare(p.codes, oc, "E4M3 codes")


def test_e4m3_encoder_negative_sample():
    """A strided sample of negative values below 512 (the sign is a separate bit)."""
    rng = np.random.default_rng(3)
    pat = np.sort(rng.integers(0, MX8_PATTERNS, 31 * 200_000, dtype=np.int64)).astype(np.uint32)
    x = np.empty((200_000, 32), np.float32)
    x[:, 0] = -256.0
    x[:, 1:] = -pat.view(np.float32).reshape(-1, 31)
    p = fp4().mxfp8_quantize(torch.from_numpy(x).to(dev()), rule="ocp")
    torch.cuda.synchronize()
    oc, os_ = oracle.mxfp8_quantize(x, oracle.MX_OCP_FLOOR)
    _compare(p.scales, os_, "E8M0 bytes")
    _compare(p.codes, oc, "E4M3 codes")


# ------------------------------------------------------------ guard bands --

CANARY = 0xA5
PAD = 4096


def _guarded(shape, dtype, ld=None):
    """A tensor of `shape` inside a larger buffer whose bytes around it (and, with
    ld > cols, between its rows) hold the canary; returns (view, buffer, mask of the
    view's own bytes)."""
    rows, cols = shape
    ld = ld or cols
    es = torch.empty((), dtype=dtype).element_size()
    nbytes = (rows * ld) * es + 2 * PAD
    buf = torch.full((nbytes,), CANARY, dtype=torch.uint8, device=dev())
    body = buf[PAD:PAD + rows * ld * es].view(dtype).view(rows, ld)
    view = body[:, :cols]
    mask = np.zeros(nbytes, bool)
    m = mask[PAD:PAD + rows * ld * es].reshape(rows, ld * es)
    m[:, :cols * es] = True
    return view, buf, mask


def _canaries_intact(buf, mask, what):
    b = buf.cpu().numpy()
    bad = np.flatnonzero((b != CANARY) & ~mask)
    assert bad.size == 0, f"{what}: {bad.size} guard bytes written, first at {bad[:4].tolist()}"


@pytest.mark.parametrize("mode", ["tensor", "row"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("rows,cols", [(1, 16), (7, 48), (33, 1040), (5, 5120), (3, 8208)])
def test_nvfp4_quantize_guard_bands(mode, dtype, rows, cols):
    from synthetic import weights

    x = torch.from_numpy(weights(rows, cols, 1.0, 0.02, 20.0, seed=rows + cols)).to(dev()).to(dtype)
    codes, cb, cm = _guarded((rows, cols // 2), torch.uint8)
    scales, sb, sm = _guarded((rows, cols // 16), torch.uint8)
    ts, tb, tm = _guarded((1, rows if mode == "row" else 1), torch.float32)
    out = fp4().PackedNVFP4(codes, scales, ts.view(-1), rows, cols, mode == "row")
    fp4().nvfp4_quantize(x, mode=mode, out=out)
    torch.cuda.synchronize()
    ref = fp4().nvfp4_quantize(x, mode=mode)
    torch.cuda.synchronize()
    assert torch.equal(codes, ref.codes) and torch.equal(scales, ref.scales) and torch.equal(ts.view(-1), ref.tscale)
    for buf, mask, what in ((cb, cm, "codes"), (sb, sm, "scales"), (tb, tm, "tensor scales")):
        _canaries_intact(buf, mask, f"nvfp4_quantize {mode} {what}")


@pytest.mark.parametrize("rows,cols", [(1, 32), (9, 96), (33, 1056), (4, 5120)])
def test_mx_quantizers_guard_bands(rows, cols):
    from synthetic import weights

    x = torch.from_numpy(weights(rows, cols, 1.0, 0.02, 20.0, seed=rows * cols)).to(dev()).to(torch.bfloat16)
    codes, cb, cm = _guarded((rows, cols // 2), torch.uint8)
    scales, sb, sm = _guarded((rows, cols // 32), torch.uint8)
    fp4().mxfp4_quantize(x, out=fp4().PackedMXFP4(codes, scales, rows, cols))
    codes8, cb8, cm8 = _guarded((rows, cols), torch.uint8)
    scales8, sb8, sm8 = _guarded((rows, cols // 32), torch.uint8)
    fp4().mxfp8_quantize(x, out=fp4().PackedMXFP8(codes8, scales8, rows, cols))
    torch.cuda.synchronize()
    r4, r8 = fp4().mxfp4_quantize(x), fp4().mxfp8_quantize(x)
    torch.cuda.synchronize()
    assert torch.equal(codes, r4.codes) and torch.equal(scales, r4.scales)
    assert torch.equal(codes8, r8.codes) and torch.equal(scales8, r8.scales)
    for buf, mask, what in ((cb, cm, "mxfp4 codes"), (sb, sm, "mxfp4 scales"), (cb8, cm8, "mxfp8 codes"),
                            (sb8, sm8, "mxfp8 scales")):
        _canaries_intact(buf, mask, what)


@pytest.mark.parametrize("ld_extra", [0, 24])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("rows,cols", [(1, 32), (9, 96), (33, 1056)])
def test_dequantizers_guard_bands(ld_extra, dtype, rows, cols):
    from synthetic import weights

    x = torch.from_numpy(weights(rows, cols, 1.0, 0.02, 20.0, seed=rows + 3 * cols)).to(dev())
    pn = fp4().nvfp4_quantize(x)
    pm = fp4().mxfp4_quantize(x)
    yn, bn, mn = _guarded((rows, cols), dtype, cols + ld_extra)
    ym, bm_, mm = _guarded((rows, cols), dtype, cols + ld_extra)
    fp4().nvfp4_dequantize(pn, dtype, out=yn)
    fp4().mxfp4_dequantize(pm, dtype, out=ym)
    torch.cuda.synchronize()
    assert torch.equal(yn, fp4().nvfp4_dequantize(pn, dtype)) and torch.equal(ym, fp4().mxfp4_dequantize(pm, dtype))
    _canaries_intact(bn, mn, f"nvfp4_dequantize ld+{ld_extra}")
    _canaries_intact(bm_, mm, f"mxfp4_dequantize ld+{ld_extra}")
