"""block_scaled_fp4_04_amd -- NVFP4 / MXFP4 block-scaled 4-bit quantization and
the quantized linear-layer GEMMs it feeds, on AMD Instinct MI355X (gfx950).

This module is a thin binding over the C ABI of ``libfp4blk.so`` (declared in
``include/fp4blk.h``): it checks tensors, hands device pointers and torch's
current stream to the library, and maps status codes to exceptions.  Every step
of the computation runs in the library's HIP kernels; there is no fallback.  If
the library is not built, importing the functions raises.

Formats ("NVFP4", newton.com.tw wiki, section "Technical principle"; edge-FP4
article, eefocus.com, section "FP4 as the next core standard"):

* NVFP4: E2M1 codes, two per byte (even column in the low nibble), one E4M3
  scale byte per 16 elements, one FP32 scale per tensor (or per row for
  dynamically quantized activations): 4.5 bits per value.
* MXFP4: E2M1 codes, one E8M0 byte per 32 elements: 4.25 bits per value.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_lib", "libfp4blk.so")

FP4_F32, FP4_BF16 = 0, 1
PER_TENSOR, PER_ROW = 0, 1
MX_OCP_FLOOR, MX_CEIL = 0, 1

_EXPORTS = {
    # name: (restype, argtypes)
}


class Fp4Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_lib = None


def _declare(L):
    p, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    sig = {
        "fp4_status_str": (ctypes.c_char_p, [i32]),
        "fp4blk_version": (i32, []),
        "fp4blk_check_device": (i32, []),
        "nvfp4_quantize_workspace": (sz, [i64, i64, i32]),
        "nvfp4_quantize": (i32, [p, i32, i64, i64, i64, p, p, p, i32, p, sz, p, p]),
        "nvfp4_dequantize": (i32, [p, p, p, i32, i64, i64, p, i32, i64, p]),
        "gemm_w4a16": (i32, [p, i64, i64, i64, p, p, p, i64, p, i32, i64, p]),
        "nvfp4_pack_decode": (i32, [p, p, i64, i64, p, p, p]),
        "gemm_w4a16_decode": (i32, [p, i64, i64, i64, p, p, p, i64, p, i32, i64, p]),
        "gemm_w4a4_workspace": (sz, [i64, i64, i32]),
        "gemm_w4a4_workspace_offsets": (None, [i64, i64, p, p, p]),
        "gemm_w4a4": (i32, [p, i64, i64, i64, i32, p, p, p, i64, p, i32, i64, p, sz, p]),
        "gemm_nvfp4_w4a4_prequant": (i32, [p, p, p, i32, i64, i64, p, p, p, i64, p, i32, i64, p]),
        "gemm_w4a4_seg": (i32, [p, i64, i64, i64, i32, p, p, p, i64, p, i32, i64, p, sz, p]),
        "gemm_nvfp4_w4a4_prequant_seg": (i32, [p, p, p, i32, i64, i64, p, p, p, i64, p, i32, i64, p]),
        "mxfp4_quantize": (i32, [p, i32, i64, i64, i64, p, p, i32, p, p]),
        "mxfp4_dequantize": (i32, [p, p, i64, i64, p, i32, i64, p]),
        "mxfp4_gemm_w4a4_workspace": (sz, [i64, i64]),
        "mxfp4_gemm_w4a4": (i32, [p, i64, i64, i64, i32, p, p, i64, p, i32, i64, p, sz, p]),
        "mxfp4_gemm_prequant": (i32, [p, p, i64, i64, p, p, i64, p, i32, i64, p]),
        "mxfp4_gemm_w4a4_seg_workspace": (sz, [i64, i64]),
        "mxfp4_gemm_w4a4_seg": (i32, [p, i64, i64, i64, i32, p, p, i64, p, i32, i64, p, sz, p]),
        "mxfp4_gemm_prequant_seg": (i32, [p, p, i64, i64, p, p, i64, p, i32, i64, p]),
        "mxfp4_gemm_w4a16": (i32, [p, i64, i64, i64, p, p, i64, p, i32, i64, p]),
        "mxfp4_pack_decode": (i32, [p, p, i64, i64, p, p, p]),
        "mxfp4_gemm_w4a16_decode": (i32, [p, i64, i64, i64, p, p, i64, p, i32, i64, p]),
        "mxfp8_quantize": (i32, [p, i32, i64, i64, i64, p, p, i32, p, p]),
        "mxfp4_gemm_w4a8_workspace": (sz, [i64, i64]),
        "mxfp4_gemm_w4a8": (i32, [p, i64, i64, i64, i32, p, p, i64, p, i32, i64, p, sz, p]),
        "mxfp4_gemm_w4a8_prequant": (i32, [p, p, i64, i64, p, p, i64, p, i32, i64, p]),
        "mxfp4_gemm_w4a8_seg": (i32, [p, i64, i64, i64, i32, p, p, i64, p, i32, i64, p, sz, p]),
        "mxfp4_gemm_w4a8_prequant_seg": (i32, [p, p, i64, i64, p, p, i64, p, i32, i64, p]),
        "nvfp4_grouped_gemm_w4a16": (i32, [p, i64, i64, i64, p, p, i64, i64, p, p, p, i64, p, i32, i64, p]),
        "mxfp4_grouped_gemm_w4a16": (i32, [p, i64, i64, i64, p, p, i64, i64, p, p, i64, p, i32, i64, p]),
        "nvfp4_grouped_gemm_w4a4_workspace": (sz, [i64, i64]),
        "nvfp4_grouped_gemm_w4a4": (i32, [p, i64, i64, i64, p, p, i64, i64, p, p, p, i64, p, i32, i64, p, sz,
                                          p]),
        "nvfp4_grouped_gemm_w4a4_prequant": (i32, [p, p, p, i64, i64, p, p, i64, i64, p, p, p, i64, p, i32,
                                                   i64, p]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return sig


def lib():
    """The loaded libfp4blk (ctypes handle).  Raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
                "(hipcc, gfx950); there is no fallback path")
        # torch first: the library links against torch's HIP runtime, which must
        # be the single HIP runtime in this process
        L = ctypes.CDLL(LIB_PATH)
        _EXPORTS.update(_declare(L))
        _lib = L
    return _lib


def exported_names():
    lib()
    return sorted(_EXPORTS)


def status_str(s: int) -> str:
    return lib().fp4_status_str(int(s)).decode()


def _check(s: int):
    if s != 0:
        raise Fp4Error(s, status_str(s))


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return FP4_F32
    if t.dtype == torch.bfloat16:
        return FP4_BF16
    raise TypeError(f"expected float32 or bfloat16, got {t.dtype}")


def _out_dt(dtype) -> int:
    return FP4_F32 if dtype == torch.float32 else FP4_BF16


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("libfp4blk takes device tensors")


def _mode(m) -> int:
    if m in ("tensor", PER_TENSOR):
        return PER_TENSOR
    if m in ("row", PER_ROW):
        return PER_ROW
    raise ValueError(f"scale mode must be 'tensor' or 'row', got {m!r}")


def _rule(r) -> int:
    if r in ("ocp", MX_OCP_FLOOR):
        return MX_OCP_FLOOR
    if r in ("ceil", MX_CEIL):
        return MX_CEIL
    raise ValueError(f"MX rule must be 'ocp' or 'ceil', got {r!r}")


def _ld(t: torch.Tensor) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit stride along its rows")
    return t.stride(0)


@dataclasses.dataclass
class PackedNVFP4:
    """NVFP4 tensor [rows, cols]: codes uint8 [rows, cols/2], scales uint8
    [rows, cols/16] (E4M3FN), tscale float32 [1] or [rows]."""
    codes: torch.Tensor
    scales: torch.Tensor
    tscale: torch.Tensor
    rows: int
    cols: int
    per_row: bool = False

    def nbytes(self) -> int:
        return self.codes.numel() + self.scales.numel() + 4 * self.tscale.numel()


@dataclasses.dataclass
class PackedMXFP4:
    """MXFP4 tensor [rows, cols]: codes uint8 [rows, cols/2], scales uint8 [rows, cols/32] (E8M0)."""
    codes: torch.Tensor
    scales: torch.Tensor
    rows: int
    cols: int

    def nbytes(self) -> int:
        return self.codes.numel() + self.scales.numel()


# --------------------------------------------------------------- NVFP4 -----

def nvfp4_quantize(x: torch.Tensor, mode="tensor", nonfinite: torch.Tensor | None = None,
                   out: PackedNVFP4 | None = None, workspace: torch.Tensor | None = None) -> PackedNVFP4:
    """Quantize a 2-D fp32/bf16 device tensor to NVFP4 (blocks along its rows)."""
    L = lib()
    _need_cuda(x, nonfinite)
    rows, cols = x.shape
    m = _mode(mode)
    dev = x.device
    if out is None:
        out = PackedNVFP4(torch.empty(rows, cols // 2, dtype=torch.uint8, device=dev),
                          torch.empty(rows, cols // 16, dtype=torch.uint8, device=dev),
                          torch.empty(rows if m == PER_ROW else 1, dtype=torch.float32, device=dev),
                          rows, cols, m == PER_ROW)
    wsb = L.nvfp4_quantize_workspace(rows, cols, m)
    if workspace is None and wsb:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=dev)
    _check(L.nvfp4_quantize(_ptr(x), _dt(x), rows, cols, _ld(x), _ptr(out.codes), _ptr(out.scales),
                            _ptr(out.tscale), m, _ptr(workspace), wsb, _ptr(nonfinite), _stream()))
    return out


def nvfp4_dequantize(p: PackedNVFP4, dtype=torch.float32, out: torch.Tensor | None = None) -> torch.Tensor:
    L = lib()
    if out is None:
        out = torch.empty(p.rows, p.cols, dtype=dtype, device=p.codes.device)
    _check(L.nvfp4_dequantize(_ptr(p.codes), _ptr(p.scales), _ptr(p.tscale),
                              PER_ROW if p.per_row else PER_TENSOR, p.rows, p.cols, _ptr(out),
                              _out_dt(out.dtype), _ld(out), _stream()))
    return out


def gemm_w4a16(a: torch.Tensor, w: PackedNVFP4, dtype=torch.bfloat16,
               out: torch.Tensor | None = None) -> torch.Tensor:
    """C = A . W^T with bf16 A [M, K] and NVFP4 W [N, K] (per-tensor scale)."""
    L = lib()
    _need_cuda(a)
    if a.dtype != torch.bfloat16:
        raise TypeError("gemm_w4a16 takes bfloat16 activations")
    M, K = a.shape
    if out is None:
        out = torch.empty(M, w.rows, dtype=dtype, device=a.device)
    _check(L.gemm_w4a16(_ptr(a), M, K, _ld(a), _ptr(w.codes), _ptr(w.scales), _ptr(w.tscale), w.rows,
                        _ptr(out), _out_dt(out.dtype), _ld(out), _stream()))
    return out


@dataclasses.dataclass
class DecodeNVFP4:
    """An NVFP4 weight [rows, cols] in the decode layout (see nvfp4_pack_decode):
    codes [cols/128, rows, 64], scales [cols/128, rows, 8], tscale [1]."""
    codes: torch.Tensor
    scales: torch.Tensor
    tscale: torch.Tensor
    rows: int
    cols: int


def nvfp4_pack_decode(w: PackedNVFP4, out: DecodeNVFP4 | None = None) -> DecodeNVFP4:
    """Rewrite a per-tensor NVFP4 weight into the decode layout (segment-major)."""
    L = lib()
    if w.per_row:
        raise ValueError("the decode layout holds weights with a per-tensor scale")
    N, K = w.rows, w.cols
    if out is None:
        dev = w.codes.device
        out = DecodeNVFP4(torch.empty(K // 128, N, 64, dtype=torch.uint8, device=dev),
                          torch.empty(K // 128, N, 8, dtype=torch.uint8, device=dev),
                          w.tscale, N, K)
    _check(L.nvfp4_pack_decode(_ptr(w.codes), _ptr(w.scales), N, K, _ptr(out.codes), _ptr(out.scales),
                               _stream()))
    return out


def gemm_w4a16_decode(a: torch.Tensor, w: DecodeNVFP4, dtype=torch.bfloat16,
                      out: torch.Tensor | None = None) -> torch.Tensor:
    """C = A . W^T for bf16 A [M, K] and W in the decode layout: the decode GEMV for M <= 16,
    the prefill GEMM on the same layout for larger M."""
    L = lib()
    _need_cuda(a)
    if a.dtype != torch.bfloat16:
        raise TypeError("gemm_w4a16_decode takes bfloat16 activations")
    M, K = a.shape
    if out is None:
        out = torch.empty(M, w.rows, dtype=dtype, device=a.device)
    _check(L.gemm_w4a16_decode(_ptr(a), M, K, _ld(a), _ptr(w.codes), _ptr(w.scales), _ptr(w.tscale), w.rows,
                               _ptr(out), _out_dt(out.dtype), _ld(out), _stream()))
    return out


def gemm_w4a4_workspace(M: int, K: int, a_mode="row", device="cuda") -> torch.Tensor:
    n = lib().gemm_w4a4_workspace(M, K, _mode(a_mode))
    return torch.empty(n, dtype=torch.uint8, device=device)


def w4a4_packed_a(ws: torch.Tensor, M: int, K: int, a_mode="row") -> PackedNVFP4:
    """Views of A's NVFP4 form inside a gemm_w4a4 workspace."""
    co, so, to = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    lib().gemm_w4a4_workspace_offsets(M, K, ctypes.byref(co), ctypes.byref(so), ctypes.byref(to))
    per_row = _mode(a_mode) == PER_ROW
    codes = ws[co.value:co.value + M * K // 2].view(M, K // 2)
    scales = ws[so.value:so.value + M * K // 16].view(M, K // 16)
    nt = M if per_row else 1
    tscale = ws[to.value:to.value + 4 * nt].view(torch.float32)
    return PackedNVFP4(codes, scales, tscale, M, K, per_row)


def gemm_w4a4(a: torch.Tensor, w: PackedNVFP4, a_mode="row", dtype=torch.bfloat16,
              out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """NVFP4 W4A4: quantize bf16 A on the device (per row by default), then C = A_q . W^T."""
    L = lib()
    _need_cuda(a)
    if a.dtype != torch.bfloat16:
        raise TypeError("gemm_w4a4 takes bfloat16 activations")
    M, K = a.shape
    m = _mode(a_mode)
    if out is None:
        out = torch.empty(M, w.rows, dtype=dtype, device=a.device)
    if workspace is None:
        workspace = gemm_w4a4_workspace(M, K, m, a.device)
    _check(L.gemm_w4a4(_ptr(a), M, K, _ld(a), m, _ptr(w.codes), _ptr(w.scales), _ptr(w.tscale), w.rows,
                       _ptr(out), _out_dt(out.dtype), _ld(out), _ptr(workspace), workspace.numel(),
                       _stream()))
    return out


def gemm_nvfp4_prequant(a: PackedNVFP4, w: PackedNVFP4, dtype=torch.bfloat16,
                        out: torch.Tensor | None = None) -> torch.Tensor:
    L = lib()
    if out is None:
        out = torch.empty(a.rows, w.rows, dtype=dtype, device=a.codes.device)
    _check(L.gemm_nvfp4_w4a4_prequant(_ptr(a.codes), _ptr(a.scales), _ptr(a.tscale),
                                      PER_ROW if a.per_row else PER_TENSOR, a.rows, a.cols,
                                      _ptr(w.codes), _ptr(w.scales), _ptr(w.tscale), w.rows, _ptr(out),
                                      _out_dt(out.dtype), _ld(out), _stream()))
    return out


def gemm_w4a4_seg(a: torch.Tensor, w: DecodeNVFP4, a_mode="row", dtype=torch.bfloat16,
                  out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """gemm_w4a4 with W in the decode layout: the same result."""
    L = lib()
    _need_cuda(a)
    if a.dtype != torch.bfloat16:
        raise TypeError("gemm_w4a4_seg takes bfloat16 activations")
    M, K = a.shape
    m = _mode(a_mode)
    if out is None:
        out = torch.empty(M, w.rows, dtype=dtype, device=a.device)
    if workspace is None:
        workspace = gemm_w4a4_workspace(M, K, m, a.device)
    _check(L.gemm_w4a4_seg(_ptr(a), M, K, _ld(a), m, _ptr(w.codes), _ptr(w.scales), _ptr(w.tscale), w.rows,
                           _ptr(out), _out_dt(out.dtype), _ld(out), _ptr(workspace), workspace.numel(), _stream()))
    return out


def gemm_nvfp4_prequant_seg(a: PackedNVFP4, w: DecodeNVFP4, dtype=torch.bfloat16,
                            out: torch.Tensor | None = None) -> torch.Tensor:
    """gemm_nvfp4_prequant with W in the decode layout."""
    L = lib()
    if out is None:
        out = torch.empty(a.rows, w.rows, dtype=dtype, device=a.codes.device)
    _check(L.gemm_nvfp4_w4a4_prequant_seg(_ptr(a.codes), _ptr(a.scales), _ptr(a.tscale),
                                          PER_ROW if a.per_row else PER_TENSOR, a.rows, a.cols,
                                          _ptr(w.codes), _ptr(w.scales), _ptr(w.tscale), w.rows, _ptr(out),
                                          _out_dt(out.dtype), _ld(out), _stream()))
    return out


# --------------------------------------------------------------- MXFP4 -----

def mxfp4_quantize(x: torch.Tensor, rule="ocp", nonfinite: torch.Tensor | None = None,
                   out: PackedMXFP4 | None = None) -> PackedMXFP4:
    L = lib()
    _need_cuda(x, nonfinite)
    rows, cols = x.shape
    if out is None:
        out = PackedMXFP4(torch.empty(rows, cols // 2, dtype=torch.uint8, device=x.device),
                          torch.empty(rows, cols // 32, dtype=torch.uint8, device=x.device), rows, cols)
    _check(L.mxfp4_quantize(_ptr(x), _dt(x), rows, cols, _ld(x), _ptr(out.codes), _ptr(out.scales),
                            _rule(rule), _ptr(nonfinite), _stream()))
    return out


def mxfp4_dequantize(p: PackedMXFP4, dtype=torch.float32, out: torch.Tensor | None = None) -> torch.Tensor:
    L = lib()
    if out is None:
        out = torch.empty(p.rows, p.cols, dtype=dtype, device=p.codes.device)
    _check(L.mxfp4_dequantize(_ptr(p.codes), _ptr(p.scales), p.rows, p.cols, _ptr(out),
                              _out_dt(out.dtype), _ld(out), _stream()))
    return out


def mxfp4_gemm_w4a4(a: torch.Tensor, w: PackedMXFP4, rule="ocp", dtype=torch.bfloat16,
                    out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    L = lib()
    _need_cuda(a)
    if a.dtype != torch.bfloat16:
        raise TypeError("mxfp4_gemm_w4a4 takes bfloat16 activations")
    M, K = a.shape
    if out is None:
        out = torch.empty(M, w.rows, dtype=dtype, device=a.device)
    if workspace is None:
        workspace = torch.empty(L.mxfp4_gemm_w4a4_workspace(M, K), dtype=torch.uint8, device=a.device)
    _check(L.mxfp4_gemm_w4a4(_ptr(a), M, K, _ld(a), _rule(rule), _ptr(w.codes), _ptr(w.scales), w.rows,
                             _ptr(out), _out_dt(out.dtype), _ld(out), _ptr(workspace), workspace.numel(),
                             _stream()))
    return out


def mxfp4_packed_a(ws: torch.Tensor, M: int, K: int) -> PackedMXFP4:
    """Views of A's MXFP4 form inside an mxfp4_gemm_w4a4 workspace."""
    cb = (M * (K // 2) + 255) // 256 * 256
    return PackedMXFP4(ws[:M * K // 2].view(M, K // 2), ws[cb:cb + M * K // 32].view(M, K // 32), M, K)


def mxfp4_gemm_prequant(a: PackedMXFP4, w: PackedMXFP4, dtype=torch.bfloat16,
                        out: torch.Tensor | None = None) -> torch.Tensor:
    L = lib()
    if out is None:
        out = torch.empty(a.rows, w.rows, dtype=dtype, device=a.codes.device)
    _check(L.mxfp4_gemm_prequant(_ptr(a.codes), _ptr(a.scales), a.rows, a.cols, _ptr(w.codes),
                                 _ptr(w.scales), w.rows, _ptr(out), _out_dt(out.dtype), _ld(out),
                                 _stream()))
    return out


def mxfp4_gemm_w4a16(a: torch.Tensor, w: PackedMXFP4, dtype=torch.bfloat16,
                     out: torch.Tensor | None = None) -> torch.Tensor:
    """C = A . W^T with bf16 A [M, K] and MXFP4 W [N, K] (K % 128 == 0)."""
    L = lib()
    _need_cuda(a)
    if a.dtype != torch.bfloat16:
        raise TypeError("mxfp4_gemm_w4a16 takes bfloat16 activations")
    M, K = a.shape
    if out is None:
        out = torch.empty(M, w.rows, dtype=dtype, device=a.device)
    _check(L.mxfp4_gemm_w4a16(_ptr(a), M, K, _ld(a), _ptr(w.codes), _ptr(w.scales), w.rows,
                              _ptr(out), _out_dt(out.dtype), _ld(out), _stream()))
    return out


@dataclasses.dataclass
class DecodeMXFP4:
    """An MXFP4 weight [rows, cols] in the decode layout (see mxfp4_pack_decode):
    codes [cols/128, rows, 64], scales [cols/128, rows, 4]."""
    codes: torch.Tensor
    scales: torch.Tensor
    rows: int
    cols: int


def mxfp4_pack_decode(w: PackedMXFP4, out: DecodeMXFP4 | None = None) -> DecodeMXFP4:
    """Rewrite an MXFP4 weight into the decode layout (segment-major)."""
    L = lib()
    N, K = w.rows, w.cols
    if out is None:
        dev = w.codes.device
        out = DecodeMXFP4(torch.empty(K // 128, N, 64, dtype=torch.uint8, device=dev),
                          torch.empty(K // 128, N, 4, dtype=torch.uint8, device=dev), N, K)
    _check(L.mxfp4_pack_decode(_ptr(w.codes), _ptr(w.scales), N, K, _ptr(out.codes), _ptr(out.scales),
                               _stream()))
    return out


def mxfp4_gemm_w4a4_seg_workspace(M: int, K: int, device="cuda") -> torch.Tensor:
    return torch.empty(lib().mxfp4_gemm_w4a4_seg_workspace(M, K), dtype=torch.uint8, device=device)


def mxfp4_seg_packed_a(ws: torch.Tensor, M: int, K: int) -> DecodeMXFP4:
    """Views of A's segment-major MXFP4 form inside an mxfp4_gemm_w4a4_seg workspace."""
    cb = (M * (K // 2) + 255) // 256 * 256
    return DecodeMXFP4(ws[:M * K // 2].view(K // 128, M, 64), ws[cb:cb + M * K // 32].view(K // 128, M, 4), M, K)


def mxfp4_gemm_w4a4_seg(a: torch.Tensor, w: DecodeMXFP4, rule="ocp", dtype=torch.bfloat16,
                        out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """MXFP4 W4A4 GEMM with W in the decode (segment-major) layout; A is quantized
    into the workspace in that layout.  The same result as mxfp4_gemm_w4a4."""
    L = lib()
    _need_cuda(a)
    if a.dtype != torch.bfloat16:
        raise TypeError("mxfp4_gemm_w4a4_seg takes bfloat16 activations")
    M, K = a.shape
    if out is None:
        out = torch.empty(M, w.rows, dtype=dtype, device=a.device)
    if workspace is None:
        workspace = mxfp4_gemm_w4a4_seg_workspace(M, K, a.device)
    _check(L.mxfp4_gemm_w4a4_seg(_ptr(a), M, K, _ld(a), _rule(rule), _ptr(w.codes), _ptr(w.scales), w.rows,
                                 _ptr(out), _out_dt(out.dtype), _ld(out), _ptr(workspace), workspace.numel(),
                                 _stream()))
    return out


def mxfp4_gemm_prequant_seg(a: DecodeMXFP4, w: DecodeMXFP4, dtype=torch.bfloat16,
                            out: torch.Tensor | None = None) -> torch.Tensor:
    """The GEMM half of mxfp4_gemm_w4a4_seg: A and W both in the segment-major layout."""
    L = lib()
    if out is None:
        out = torch.empty(a.rows, w.rows, dtype=dtype, device=a.codes.device)
    _check(L.mxfp4_gemm_prequant_seg(_ptr(a.codes), _ptr(a.scales), a.rows, a.cols, _ptr(w.codes),
                                     _ptr(w.scales), w.rows, _ptr(out), _out_dt(out.dtype), _ld(out), _stream()))
    return out


def mxfp4_gemm_w4a16_decode(a: torch.Tensor, w: DecodeMXFP4, dtype=torch.bfloat16,
                            out: torch.Tensor | None = None) -> torch.Tensor:
    """C = A . W^T for bf16 A [M, K] and an MXFP4 W in the decode layout (GEMV for M <= 16,
    the prefill GEMM on the same layout for larger M)."""
    L = lib()
    _need_cuda(a)
    if a.dtype != torch.bfloat16:
        raise TypeError("mxfp4_gemm_w4a16_decode takes bfloat16 activations")
    M, K = a.shape
    if out is None:
        out = torch.empty(M, w.rows, dtype=dtype, device=a.device)
    _check(L.mxfp4_gemm_w4a16_decode(_ptr(a), M, K, _ld(a), _ptr(w.codes), _ptr(w.scales), w.rows,
                                     _ptr(out), _out_dt(out.dtype), _ld(out), _stream()))
    return out


@dataclasses.dataclass
class PackedMXFP8:
    """An MXFP8 tensor [rows, cols]: E4M3FN codes [rows, cols], E8M0 scales [rows, cols/32]."""
    codes: torch.Tensor
    scales: torch.Tensor
    rows: int
    cols: int


def mxfp8_quantize(x: torch.Tensor, rule="ocp", nonfinite: torch.Tensor | None = None,
                   out: PackedMXFP8 | None = None) -> PackedMXFP8:
    """MXFP8 (E4M3FN elements, E8M0 per 32) of an fp32 or bf16 [rows, cols] tensor."""
    L = lib()
    _need_cuda(x)
    rows, cols = x.shape
    if out is None:
        out = PackedMXFP8(torch.empty(rows, cols, dtype=torch.uint8, device=x.device),
                          torch.empty(rows, cols // 32, dtype=torch.uint8, device=x.device), rows, cols)
    _check(L.mxfp8_quantize(_ptr(x), _dt(x), rows, cols, _ld(x), _ptr(out.codes), _ptr(out.scales),
                            _rule(rule), _ptr(nonfinite), _stream()))
    return out


def mxfp4_gemm_w4a8_workspace(M: int, K: int, device="cuda") -> torch.Tensor:
    return torch.empty(lib().mxfp4_gemm_w4a8_workspace(M, K), dtype=torch.uint8, device=device)


def mxfp8_packed_a(ws: torch.Tensor, M: int, K: int) -> PackedMXFP8:
    """A's MXFP8 form inside a mxfp4_gemm_w4a8 workspace."""
    cb = (M * K + 255) // 256 * 256
    return PackedMXFP8(ws[:M * K].view(M, K), ws[cb:cb + M * K // 32].view(M, K // 32), M, K)


def mxfp4_gemm_w4a8(a: torch.Tensor, w: PackedMXFP4, rule="ocp", dtype=torch.bfloat16,
                    out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """W4A8: bf16 A [M, K] quantized to MXFP8 on the device, MXFP4 W [N, K]."""
    L = lib()
    _need_cuda(a)
    if a.dtype != torch.bfloat16:
        raise TypeError("mxfp4_gemm_w4a8 takes bfloat16 activations")
    M, K = a.shape
    if workspace is None:
        workspace = mxfp4_gemm_w4a8_workspace(M, K, a.device)
    if out is None:
        out = torch.empty(M, w.rows, dtype=dtype, device=a.device)
    _check(L.mxfp4_gemm_w4a8(_ptr(a), M, K, _ld(a), _rule(rule), _ptr(w.codes), _ptr(w.scales), w.rows,
                             _ptr(out), _out_dt(out.dtype), _ld(out), _ptr(workspace), workspace.numel(),
                             _stream()))
    return out


def mxfp4_gemm_w4a8_prequant(a: PackedMXFP8, w: PackedMXFP4, dtype=torch.bfloat16,
                             out: torch.Tensor | None = None) -> torch.Tensor:
    """The GEMM half of mxfp4_gemm_w4a8 on an MXFP8 A."""
    L = lib()
    if out is None:
        out = torch.empty(a.rows, w.rows, dtype=dtype, device=a.codes.device)
    _check(L.mxfp4_gemm_w4a8_prequant(_ptr(a.codes), _ptr(a.scales), a.rows, a.cols, _ptr(w.codes),
                                      _ptr(w.scales), w.rows, _ptr(out), _out_dt(out.dtype), _ld(out),
                                      _stream()))
    return out


def mxfp4_gemm_w4a8_seg(a: torch.Tensor, w: DecodeMXFP4, rule="ocp", dtype=torch.bfloat16,
                        out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """W4A8 with the MXFP4 W in the decode (segment-major) layout; the same result as mxfp4_gemm_w4a8."""
    L = lib()
    _need_cuda(a)
    if a.dtype != torch.bfloat16:
        raise TypeError("mxfp4_gemm_w4a8_seg takes bfloat16 activations")
    M, K = a.shape
    if workspace is None:
        workspace = mxfp4_gemm_w4a8_workspace(M, K, a.device)
    if out is None:
        out = torch.empty(M, w.rows, dtype=dtype, device=a.device)
    _check(L.mxfp4_gemm_w4a8_seg(_ptr(a), M, K, _ld(a), _rule(rule), _ptr(w.codes), _ptr(w.scales), w.rows,
                                 _ptr(out), _out_dt(out.dtype), _ld(out), _ptr(workspace), workspace.numel(),
                                 _stream()))
    return out


def mxfp4_gemm_w4a8_prequant_seg(a: PackedMXFP8, w: DecodeMXFP4, dtype=torch.bfloat16,
                                 out: torch.Tensor | None = None) -> torch.Tensor:
    """The GEMM half of mxfp4_gemm_w4a8_seg on an MXFP8 A."""
    L = lib()
    if out is None:
        out = torch.empty(a.rows, w.rows, dtype=dtype, device=a.codes.device)
    _check(L.mxfp4_gemm_w4a8_prequant_seg(_ptr(a.codes), _ptr(a.scales), a.rows, a.cols, _ptr(w.codes),
                                          _ptr(w.scales), w.rows, _ptr(out), _out_dt(out.dtype), _ld(out),
                                          _stream()))
    return out


# ------------------------------------------------------- grouped (MoE) -----

@dataclasses.dataclass
class ExpertsNVFP4:
    """E NVFP4 expert weights [E, N, K]: codes uint8 [E, N, K/2], scales uint8
    [E, N, K/16], one float32 tensor scale per expert [E]."""
    codes: torch.Tensor
    scales: torch.Tensor
    tscale: torch.Tensor
    experts: int
    rows: int
    cols: int


@dataclasses.dataclass
class ExpertsMXFP4:
    """E MXFP4 expert weights [E, N, K]: codes uint8 [E, N, K/2], scales uint8 [E, N, K/32]."""
    codes: torch.Tensor
    scales: torch.Tensor
    experts: int
    rows: int
    cols: int


def nvfp4_quantize_experts(w: torch.Tensor) -> ExpertsNVFP4:
    """Each expert of w [E, N, K] quantized as its own NVFP4 tensor (its own tensor scale)."""
    E, N, K = w.shape
    dev = w.device
    out = ExpertsNVFP4(torch.empty(E, N, K // 2, dtype=torch.uint8, device=dev),
                       torch.empty(E, N, K // 16, dtype=torch.uint8, device=dev),
                       torch.empty(E, dtype=torch.float32, device=dev), E, N, K)
    ws = torch.empty(max(1, lib().nvfp4_quantize_workspace(N, K, PER_TENSOR)), dtype=torch.uint8, device=dev)
    for e in range(E):
        nvfp4_quantize(w[e], out=PackedNVFP4(out.codes[e], out.scales[e], out.tscale[e:e + 1], N, K),
                       workspace=ws)
    return out


def mxfp4_quantize_experts(w: torch.Tensor, rule="ocp") -> ExpertsMXFP4:
    """MXFP4 of expert weights w [E, N, K] (blocks along K; no tensor scale)."""
    E, N, K = w.shape
    p = mxfp4_quantize(w.reshape(E * N, K), rule=rule)
    return ExpertsMXFP4(p.codes.view(E, N, K // 2), p.scales.view(E, N, K // 32), E, N, K)


def _grouped_common(a_rows, group_offs, row_index):
    _need_cuda(group_offs, row_index)
    if group_offs.dtype != torch.int32 or not group_offs.is_contiguous():
        raise TypeError("group_offs must be a contiguous int32 device tensor [groups + 1]")
    if row_index is not None and (row_index.dtype != torch.int32 or not row_index.is_contiguous()):
        raise TypeError("row_index must be a contiguous int32 device tensor [rows]")
    rows = row_index.numel() if row_index is not None else a_rows
    return rows, group_offs.numel() - 1


def nvfp4_grouped_gemm_w4a16(a: torch.Tensor, w: ExpertsNVFP4, group_offs: torch.Tensor,
                             row_index: torch.Tensor | None = None, dtype=torch.bfloat16,
                             out: torch.Tensor | None = None) -> torch.Tensor:
    """C[t] = A[row_index[t]] . W_e^T for the grouped rows t of group e (bf16 A, NVFP4 experts)."""
    L = lib()
    _need_cuda(a)
    rows, groups = _grouped_common(a.shape[0], group_offs, row_index)
    if out is None:
        out = torch.empty(rows, w.rows, dtype=dtype, device=a.device)
    _check(L.nvfp4_grouped_gemm_w4a16(_ptr(a), a.shape[0], a.shape[1], _ld(a), _ptr(row_index), _ptr(group_offs),
                                      groups, rows, _ptr(w.codes), _ptr(w.scales), _ptr(w.tscale), w.rows,
                                      _ptr(out), _out_dt(out.dtype), _ld(out), _stream()))
    return out


def mxfp4_grouped_gemm_w4a16(a: torch.Tensor, w: ExpertsMXFP4, group_offs: torch.Tensor,
                             row_index: torch.Tensor | None = None, dtype=torch.bfloat16,
                             out: torch.Tensor | None = None) -> torch.Tensor:
    """As nvfp4_grouped_gemm_w4a16 with MXFP4 experts."""
    L = lib()
    _need_cuda(a)
    rows, groups = _grouped_common(a.shape[0], group_offs, row_index)
    if out is None:
        out = torch.empty(rows, w.rows, dtype=dtype, device=a.device)
    _check(L.mxfp4_grouped_gemm_w4a16(_ptr(a), a.shape[0], a.shape[1], _ld(a), _ptr(row_index), _ptr(group_offs),
                                      groups, rows, _ptr(w.codes), _ptr(w.scales), w.rows, _ptr(out),
                                      _out_dt(out.dtype), _ld(out), _stream()))
    return out


def nvfp4_grouped_gemm_w4a4_workspace(a_rows: int, K: int, device="cuda") -> torch.Tensor:
    return torch.empty(lib().nvfp4_grouped_gemm_w4a4_workspace(a_rows, K), dtype=torch.uint8, device=device)


def nvfp4_grouped_gemm_w4a4(a: torch.Tensor, w: ExpertsNVFP4, group_offs: torch.Tensor,
                            row_index: torch.Tensor | None = None, dtype=torch.bfloat16,
                            out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """NVFP4 W4A4 grouped GEMM: every A row quantized once per row, then gathered per group."""
    L = lib()
    _need_cuda(a)
    if a.dtype != torch.bfloat16:
        raise TypeError("nvfp4_grouped_gemm_w4a4 takes bfloat16 activations")
    rows, groups = _grouped_common(a.shape[0], group_offs, row_index)
    if workspace is None:
        workspace = nvfp4_grouped_gemm_w4a4_workspace(a.shape[0], a.shape[1], a.device)
    if out is None:
        out = torch.empty(rows, w.rows, dtype=dtype, device=a.device)
    _check(L.nvfp4_grouped_gemm_w4a4(_ptr(a), a.shape[0], a.shape[1], _ld(a), _ptr(row_index), _ptr(group_offs),
                                     groups, rows, _ptr(w.codes), _ptr(w.scales), _ptr(w.tscale), w.rows,
                                     _ptr(out), _out_dt(out.dtype), _ld(out), _ptr(workspace), workspace.numel(),
                                     _stream()))
    return out


def nvfp4_grouped_gemm_w4a4_prequant(a: PackedNVFP4, w: ExpertsNVFP4, group_offs: torch.Tensor,
                                     row_index: torch.Tensor | None = None, dtype=torch.bfloat16,
                                     out: torch.Tensor | None = None) -> torch.Tensor:
    """The GEMM half of nvfp4_grouped_gemm_w4a4 on a per-row NVFP4 A."""
    L = lib()
    if not a.per_row:
        raise ValueError("the grouped W4A4 GEMM takes a per-row NVFP4 A")
    rows, groups = _grouped_common(a.rows, group_offs, row_index)
    if out is None:
        out = torch.empty(rows, w.rows, dtype=dtype, device=a.codes.device)
    _check(L.nvfp4_grouped_gemm_w4a4_prequant(_ptr(a.codes), _ptr(a.scales), _ptr(a.tscale), a.rows, a.cols,
                                              _ptr(row_index), _ptr(group_offs), groups, rows, _ptr(w.codes),
                                              _ptr(w.scales), _ptr(w.tscale), w.rows, _ptr(out),
                                              _out_dt(out.dtype), _ld(out), _stream()))
    return out
