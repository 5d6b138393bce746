"""GPU parity of the quantizers and dequantizers past 2^32 elements.

NVFP4 (NVFP4 wiki, format section: E2M1 values, E4M3 scale per 16, fp32 tensor
scale) and MXFP4 / MXFP8 (edge-FP4 article, section "FP4 as the next core
standard": E8M0 scale per 32).  One bf16 tensor of 838,898 x 5120 =
4,295,157,760 elements (8.6 GB; 17.2 GB as fp32), so that the element index
passes 2^31 and 2^32, the bf16 input's byte offset passes 2^32 and 2^33, the
fp32 input's passes 2^34, and the FP4 codes' byte offset passes 2^31.  The
column count makes the row divider a non-power of two (640 units of 8).

Input: 97 seeded rows of activations, row r being base row r % 97 times
2^(((r // 97) % 7) - 3), an exact scaling in bf16, built on the device in row
chunks.  The oracle quantizes the sampled rows rebuilt on the host; the sample
holds the rows where each of those offsets is crossed, the first and last
rows, random rows, and a row holding the tensor's largest magnitude, so the
oracle's per-tensor scale over the sample equals the scale over the whole
tensor.  Codes, scale bytes and tensor scales must be equal bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import bf16bits_to_dev, bf16_tensor_bits, dev, log
from synthetic import activations_f32, bf16_bits_to_f32, to_bf16_bits

pytestmark = pytest.mark.gpu

P = 97
COLS = 5120
ROWS = (1 << 32) // COLS + 38          # 838,898
CHUNK = 65536


def fp4():
    import block_scaled_fp4_04_amd as m

    return m


def _exp(r):
    return ((np.asarray(r) // P) % 7) - 3


@pytest.fixture(scope="module")
def big():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    assert ROWS * COLS > (1 << 32)
    base_bits = to_bf16_bits(activations_f32(P, COLS, 0.005, 30.0, seed=31))
    log(f"building the bf16 input {ROWS}x{COLS} on the device")
    base = bf16bits_to_dev(base_bits)
    x = torch.empty(ROWS, COLS, dtype=torch.bfloat16, device=dev())
    for r0 in range(0, ROWS, CHUNK):
        r = torch.arange(r0, min(ROWS, r0 + CHUNK), device=dev())
        f = torch.exp2((torch.div(r, P, rounding_mode="floor") % 7 - 3).float()).to(torch.bfloat16)
        x[r0:r0 + r.numel()] = base[r % P] * f[:, None]
    torch.cuda.synchronize()
    pstar = int(np.argmax(np.abs(bf16_bits_to_f32(base_bits)).max(axis=1)))
    r_max = P * 6 + pstar                 # exponent +3: a row holding the tensor's amax
    assert _exp(r_max) == 3
    cross = []
    for elem in (1 << 29, 1 << 30, 1 << 31, 1 << 32):   # fp32 2^31 B, bf16 2^31 B, 2^31 / 2^32 elements
        r = elem // COLS
        cross += [r - 1, r, r + 1]
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, P - 1, r_max, ROWS - 2, ROWS - 1], cross,
                                     rng.choice(ROWS, 8, replace=False)]))
    assert rows.max() < ROWS
    host = np.stack([to_bf16_bits(bf16_bits_to_f32(base_bits[r % P]) * np.float32(2.0 ** _exp(r)))
                     for r in rows])
    # the device rows are the host rows (the construction is exact)
    ri = torch.from_numpy(rows).to(dev())
    assert np.array_equal(bf16_tensor_bits(x[ri]), host)
    yield x, rows, ri, host
    del x, base
    torch.cuda.empty_cache()


def _rows(t, ri):
    return t[ri].cpu().numpy()


@pytest.mark.parametrize("mode", ["row", "tensor"])
def test_nvfp4_quantize_dequantize_past_2e32(big, mode):
    x, rows, ri, host = big
    per_row = mode == "row"
    log(f"nvfp4_quantize {ROWS}x{COLS} bf16 mode={mode}")
    p = fp4().nvfp4_quantize(x, mode=mode)
    torch.cuda.synchronize()
    oc, os_, ot = oracle.nvfp4_quantize(host, per_row=per_row)
    assert np.array_equal(_rows(p.codes, ri), oc)
    assert np.array_equal(_rows(p.scales, ri), os_)
    got_t = _rows(p.tscale, ri) if per_row else p.tscale.cpu().numpy()
    assert np.array_equal(got_t.view(np.uint32), ot.view(np.uint32))
    log(f"nvfp4_dequantize {ROWS}x{COLS} -> bf16 mode={mode}")
    y = fp4().nvfp4_dequantize(p, torch.bfloat16)
    torch.cuda.synchronize()
    want = oracle.f32_to_bf16_bits(oracle.nvfp4_dequantize(oc, os_, ot, per_row=per_row))
    assert np.array_equal(bf16_tensor_bits(y[ri]), want)
    del p, y
    torch.cuda.empty_cache()


def test_nvfp4_quantize_fp32_input_past_2e34_bytes(big):
    x, rows, ri, host = big
    log(f"nvfp4_quantize {ROWS}x{COLS} fp32 (17.2 GB input) mode=tensor")
    x32 = torch.empty(ROWS, COLS, dtype=torch.float32, device=dev())
    for r0 in range(0, ROWS, CHUNK):
        x32[r0:r0 + CHUNK] = x[r0:r0 + CHUNK].float()
    p = fp4().nvfp4_quantize(x32)
    torch.cuda.synchronize()
    oc, os_, ot = oracle.nvfp4_quantize(bf16_bits_to_f32(host))
    assert np.array_equal(_rows(p.codes, ri), oc)
    assert np.array_equal(_rows(p.scales, ri), os_)
    assert np.array_equal(p.tscale.cpu().numpy().view(np.uint32), ot.view(np.uint32))
    del x32, p
    torch.cuda.empty_cache()


def test_mxfp4_quantize_dequantize_past_2e32(big):
    x, rows, ri, host = big
    log(f"mxfp4_quantize {ROWS}x{COLS} bf16 rule=ocp")
    p = fp4().mxfp4_quantize(x)
    torch.cuda.synchronize()
    oc, os_ = oracle.mxfp4_quantize(host)
    assert np.array_equal(_rows(p.codes, ri), oc)
    assert np.array_equal(_rows(p.scales, ri), os_)
    log(f"mxfp4_dequantize {ROWS}x{COLS} -> bf16")
    y = fp4().mxfp4_dequantize(p, torch.bfloat16)
    torch.cuda.synchronize()
    want = oracle.f32_to_bf16_bits(oracle.mxfp4_dequantize(oc, os_))
    assert np.array_equal(bf16_tensor_bits(y[ri]), want)
    del p, y
    torch.cuda.empty_cache()


def test_mxfp8_quantize_past_2e32(big):
    x, rows, ri, host = big
    log(f"mxfp8_quantize {ROWS}x{COLS} bf16 rule=ocp (4.3 GB of codes)")
    p = fp4().mxfp8_quantize(x)
    torch.cuda.synchronize()
    oc, os_ = oracle.mxfp8_quantize(host)
    assert np.array_equal(_rows(p.codes, ri), oc)
    assert np.array_equal(_rows(p.scales, ri), os_)
    del p
    torch.cuda.empty_cache()
