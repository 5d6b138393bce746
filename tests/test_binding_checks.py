"""Host checks of the Python binding's argument validation (no GPU needed).

The C ABI receives bare pointers and sizes, so a tensor smaller than the sizes
passed with it would be read or written past its end.  The binding therefore
checks every tensor's shape, dtype and layout against the call before anything
reaches the library, and only then that all tensors are device tensors on one
device.  These tests pass host tensors: a mismatch must raise its own error, and
a well-formed call must get as far as the device check.
"""
import pytest
import torch

import block_scaled_fp4_04_amd as fp4

U8, F32, BF16 = torch.uint8, torch.float32, torch.bfloat16


def nv(rows, cols, per_row=False):
    return fp4.PackedNVFP4(torch.zeros(rows, cols // 2, dtype=U8), torch.zeros(rows, cols // 16, dtype=U8),
                           torch.zeros(rows if per_row else 1, dtype=F32), rows, cols, per_row)


def mx(rows, cols):
    return fp4.PackedMXFP4(torch.zeros(rows, cols // 2, dtype=U8), torch.zeros(rows, cols // 32, dtype=U8),
                           rows, cols)


def nv_dec(rows, cols):
    return fp4.DecodeNVFP4(torch.zeros(cols // 128, rows, 64, dtype=U8), torch.zeros(cols // 128, rows, 8, dtype=U8),
                           torch.zeros(1, dtype=F32), rows, cols)


def mx_dec(rows, cols):
    return fp4.DecodeMXFP4(torch.zeros(cols // 128, rows, 64, dtype=U8), torch.zeros(cols // 128, rows, 4, dtype=U8),
                           rows, cols)


def a16(M, K):
    return torch.zeros(M, K, dtype=BF16)


def reaches_device_check(fn, *args, **kw):
    with pytest.raises(ValueError, match="device tensors"):
        fn(*args, **kw)


# --------------------------------------------------------- well-formed calls

def test_well_formed_calls_reach_the_device_check():
    reaches_device_check(fp4.gemm_w4a16, a16(4, 256), nv(64, 256))
    reaches_device_check(fp4.gemm_w4a16, a16(4, 256), nv(64, 256), out=torch.zeros(4, 64, dtype=F32))
    reaches_device_check(fp4.gemm_w4a4, a16(4, 256), nv(64, 256))
    reaches_device_check(fp4.gemm_w4a16_decode, a16(4, 256), nv_dec(64, 256))
    reaches_device_check(fp4.mxfp4_gemm_w4a4, a16(4, 256), mx(64, 256))
    reaches_device_check(fp4.mxfp4_gemm_w4a16_decode, a16(4, 256), mx_dec(64, 256))
    reaches_device_check(fp4.mxfp4_gemm_w4a8_seg, a16(4, 256), mx_dec(64, 256))
    reaches_device_check(fp4.nvfp4_quantize, torch.zeros(8, 64))
    reaches_device_check(fp4.nvfp4_dequantize, nv(8, 64), out=torch.zeros(8, 64, dtype=BF16))
    reaches_device_check(fp4.mxfp4_dequantize, mx(8, 64))
    reaches_device_check(fp4.gemm_nvfp4_prequant, nv(4, 256, per_row=True), nv(64, 256))


# ------------------------------------------------------------ K mismatch ---

@pytest.mark.parametrize("call", [
    lambda: fp4.gemm_w4a16(a16(4, 256), nv(64, 128)),
    lambda: fp4.gemm_w4a4(a16(4, 256), nv(64, 512)),
    lambda: fp4.gemm_w4a4_seg(a16(4, 256), nv_dec(64, 384)),
    lambda: fp4.gemm_w4a16_decode(a16(1, 256), nv_dec(64, 128)),
    lambda: fp4.gemm_nvfp4_prequant(nv(4, 256, True), nv(64, 128)),
    lambda: fp4.gemm_nvfp4_prequant_seg(nv(4, 256, True), nv_dec(64, 128)),
    lambda: fp4.mxfp4_gemm_w4a4(a16(4, 256), mx(64, 128)),
    lambda: fp4.mxfp4_gemm_w4a16(a16(4, 256), mx(64, 128)),
    lambda: fp4.mxfp4_gemm_w4a16_decode(a16(4, 256), mx_dec(64, 128)),
    lambda: fp4.mxfp4_gemm_prequant(mx(4, 256), mx(64, 128)),
    lambda: fp4.mxfp4_gemm_w4a8(a16(4, 256), mx(64, 128)),
])
def test_k_mismatch_is_refused(call):
    with pytest.raises(ValueError, match="K = "):
        call()


# ----------------------------------------------------------- bad outputs ---

@pytest.mark.parametrize("out", [
    torch.zeros(3, 64, dtype=F32),          # too few rows
    torch.zeros(4, 63, dtype=F32),          # too few columns
    torch.zeros(4, 65, dtype=BF16),         # too many columns
    torch.zeros(4 * 64, dtype=F32),         # not 2-D
    torch.zeros(64, 4, dtype=F32).t(),      # column-major
])
def test_out_shape_and_layout_are_checked(out):
    with pytest.raises(ValueError):
        fp4.gemm_w4a16(a16(4, 256), nv(64, 256), out=out)


@pytest.mark.parametrize("dtype", [torch.float16, torch.float64, torch.int32])
def test_out_dtype_is_checked(dtype):
    with pytest.raises(TypeError):
        fp4.gemm_w4a16(a16(4, 256), nv(64, 256), out=torch.zeros(4, 64, dtype=dtype))
    with pytest.raises(TypeError):
        fp4.gemm_w4a16(a16(4, 256), nv(64, 256), dtype=dtype)
    with pytest.raises(TypeError):
        fp4.nvfp4_dequantize(nv(8, 64), dtype)


def test_dequantize_out_is_checked():
    with pytest.raises(ValueError):
        fp4.nvfp4_dequantize(nv(8, 64), out=torch.zeros(7, 64))
    with pytest.raises(ValueError):
        fp4.mxfp4_dequantize(mx(8, 64), out=torch.zeros(8, 32))


# ------------------------------------------------- packed operand sizes ----

def test_packed_sizes_are_checked():
    w = nv(64, 256)
    w.codes = torch.zeros(64, 100, dtype=U8)
    with pytest.raises(ValueError, match="codes"):
        fp4.gemm_w4a16(a16(4, 256), w)
    w = nv(64, 256)
    w.scales = torch.zeros(63, 16, dtype=U8)
    with pytest.raises(ValueError, match="scales"):
        fp4.gemm_w4a16(a16(4, 256), w)
    w = nv(64, 256)
    w.codes = torch.zeros(64, 128, dtype=torch.int8)
    with pytest.raises(TypeError):
        fp4.gemm_w4a16(a16(4, 256), w)
    w = nv(64, 256)
    w.codes = torch.zeros(128, 64, dtype=U8).t()
    with pytest.raises(ValueError, match="contiguous"):
        fp4.gemm_w4a16(a16(4, 256), w)
    m = mx(64, 256)
    m.scales = torch.zeros(64, 4, dtype=U8)
    with pytest.raises(ValueError, match="scales"):
        fp4.mxfp4_gemm_w4a4(a16(4, 256), m)
    d = nv_dec(64, 256)
    d.codes = torch.zeros(2, 63, 64, dtype=U8)
    with pytest.raises(ValueError, match="codes"):
        fp4.gemm_w4a16_decode(a16(1, 256), d)


def test_tensor_scale_sizes_are_checked():
    w = nv(64, 256)
    w.tscale = torch.zeros(2, dtype=F32)
    with pytest.raises(ValueError, match="tensor scale"):
        fp4.gemm_w4a16(a16(4, 256), w)
    a = nv(4, 256, per_row=True)
    a.tscale = torch.zeros(3, dtype=F32)
    with pytest.raises(ValueError, match="tensor scale"):
        fp4.gemm_nvfp4_prequant(a, nv(64, 256))
    with pytest.raises(ValueError, match="one tensor scale"):
        fp4.gemm_w4a16(a16(4, 256), nv(64, 256, per_row=True))


def test_quantize_outputs_are_checked():
    x = torch.zeros(8, 64)
    with pytest.raises(ValueError, match="does not describe"):
        fp4.nvfp4_quantize(x, out=nv(8, 32))
    with pytest.raises(ValueError, match="does not describe"):
        fp4.nvfp4_quantize(x, mode="row", out=nv(8, 64))
    bad = nv(8, 64)
    bad.scales = torch.zeros(8, 3, dtype=U8)
    with pytest.raises(ValueError, match="scales"):
        fp4.nvfp4_quantize(x, out=bad)
    with pytest.raises(ValueError, match="does not describe"):
        fp4.mxfp4_quantize(x, out=mx(4, 64))
    with pytest.raises(ValueError, match="does not describe"):
        fp4.mxfp8_quantize(x, out=fp4.PackedMXFP8(torch.zeros(8, 64, dtype=U8), torch.zeros(8, 2, dtype=U8), 8, 32))
    with pytest.raises(ValueError, match="nonfinite"):
        fp4.nvfp4_quantize(x, nonfinite=torch.zeros(1, dtype=torch.int64))


def test_workspace_is_checked():
    with pytest.raises(ValueError, match="workspace"):
        fp4.gemm_w4a4(a16(4, 256), nv(64, 256), workspace=torch.zeros(16, dtype=U8))
    with pytest.raises(ValueError, match="workspace"):
        fp4.mxfp4_gemm_w4a4(a16(4, 256), mx(64, 256), workspace=torch.zeros(10, 10, dtype=U8))
    with pytest.raises(ValueError, match="workspace"):
        fp4.nvfp4_quantize(torch.zeros(8, 64), workspace=torch.zeros(4, dtype=U8))


def test_activation_dtype_and_rank_are_checked():
    with pytest.raises(TypeError):
        fp4.gemm_w4a16(torch.zeros(4, 256, dtype=F32), nv(64, 256))
    with pytest.raises(ValueError):
        fp4.gemm_w4a16(torch.zeros(2, 4, 256, dtype=BF16), nv(64, 256))
    with pytest.raises(TypeError):
        fp4.nvfp4_quantize(torch.zeros(8, 64, dtype=torch.float16))


def test_grouped_arguments_are_checked():
    E, N, K = 3, 64, 256
    w = fp4.ExpertsNVFP4(torch.zeros(E, N, K // 2, dtype=U8), torch.zeros(E, N, K // 16, dtype=U8),
                         torch.zeros(E, dtype=F32), E, N, K)
    offs = torch.tensor([0, 2, 3, 4], dtype=torch.int32)
    reaches_device_check(fp4.nvfp4_grouped_gemm_w4a16, a16(4, K), w, offs)
    with pytest.raises(ValueError, match="experts"):
        fp4.nvfp4_grouped_gemm_w4a16(a16(4, K), w, torch.tensor([0, 2, 4], dtype=torch.int32))
    with pytest.raises(ValueError, match="K = "):
        fp4.nvfp4_grouped_gemm_w4a16(a16(4, 128), w, offs)
    with pytest.raises(TypeError):
        fp4.nvfp4_grouped_gemm_w4a16(a16(4, K), w, offs.long())
    with pytest.raises(ValueError, match="out"):
        fp4.nvfp4_grouped_gemm_w4a4(a16(4, K), w, offs, out=torch.zeros(3, N))
    short = fp4.ExpertsNVFP4(w.codes[:2], w.scales, w.tscale, E, N, K)
    with pytest.raises(ValueError, match="codes"):
        fp4.nvfp4_grouped_gemm_w4a16(a16(4, K), short, offs)
    m = fp4.ExpertsMXFP4(torch.zeros(E, N, K // 2, dtype=U8), torch.zeros(E, N, K // 16, dtype=U8), E, N, K)
    with pytest.raises(ValueError, match="scales"):
        fp4.mxfp4_grouped_gemm_w4a16(a16(4, K), m, offs)


def test_single_row_stride_is_the_row_length():
    x = torch.zeros(128)[None, :]                      # unsqueeze: row stride 0
    assert fp4._ld(x) == 128
    assert fp4._ld(torch.zeros(1, 64).expand(1, 64)) == 64
    assert fp4._ld(torch.zeros(3, 256)[:, :64]) == 256
    with pytest.raises(ValueError):
        fp4._ld(torch.zeros(64, 4).t())
