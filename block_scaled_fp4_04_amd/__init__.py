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
        "fp4blk_read_ceiling": (i32, [p, sz, i32, p, p]),
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
        "gemm_w4a4_noalloc": (i32, [p, i64, i64, i64, i32, p, p, p, i64, p, i32, i64, p]),
        "gemm_nvfp4_w4a4_prequant_seg": (i32, [p, p, p, i32, i64, i64, p, p, p, i64, p, i32, i64, p]),
        "mxfp4_quantize": (i32, [p, i32, i64, i64, i64, p, p, i32, p, p]),
        "mxfp4_dequantize": (i32, [p, p, i64, i64, p, i32, i64, p]),
        "mxfp4_gemm_w4a4_workspace": (sz, [i64, i64]),
        "mxfp4_gemm_w4a4_a_segment_major": (i32, [i64, i64, i64]),
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


_recording = None  # list of (function, arguments) while prepare() records
_recording_keep = []  # the tensors behind the recorded pointers


def _run(fn, *args):
    """Every library call goes through here: made at once, or recorded by prepare()."""
    if _recording is not None:
        _recording.append((fn, args))
        return
    _check(fn(*args))


class Prepared:
    """Library calls recorded by prepare(), replayed with the same pointers, sizes and
    stream.  It holds the tensors the calls use, so their memory stays valid."""

    def __init__(self, calls, keep):
        self._calls = calls
        self._keep = keep

    def __call__(self, *_ignored):
        for fn, args in self._calls:
            s = fn(*args)
            if s != 0:
                raise Fp4Error(s, status_str(s))


def prepare(thunk, *keep) -> Prepared:
    """Runs `thunk` (one or more calls of this module) with every argument check made
    and the library calls recorded instead of launched, and returns a callable that
    launches exactly those calls again: the same device pointers, sizes and stream,
    without the Python-side checks and allocation.  For tight loops (decode steps,
    benchmarks) where the checks would cost more than a short kernel.  The callable
    holds every tensor whose memory the calls use (and what the thunk returns), so
    that memory stays valid; the tensors' contents may change between calls."""
    global _recording, _recording_keep
    if _recording is not None:
        raise RuntimeError("prepare() calls do not nest")
    _recording, _recording_keep = [], []
    try:
        result = thunk()
        calls, held = _recording, _recording_keep
    finally:
        _recording, _recording_keep = None, []
    return Prepared(calls, (result, keep, held))


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    if t is not None and _recording is not None:
        _recording_keep.append(t)  # prepare(): the replayed calls keep using this memory
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return FP4_F32
    if t.dtype == torch.bfloat16:
        return FP4_BF16
    raise TypeError(f"expected float32 or bfloat16, got {t.dtype}")


def _out_dt(dtype) -> int:
    if dtype == torch.float32:
        return FP4_F32
    if dtype == torch.bfloat16:
        return FP4_BF16
    raise TypeError(f"outputs are float32 or bfloat16, got {dtype}")


def _need_cuda(*ts):
    """Every tensor given is a device tensor, and all are on one device."""
    devs = {t.device for t in ts if t is not None}
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("libfp4blk takes device tensors")
    if len(devs) > 1:
        raise ValueError(f"tensors on several devices: {sorted(str(d) for d in devs)}")


# Argument checks.  The C ABI receives bare pointers and sizes, so it cannot see a
# tensor that is smaller than the sizes passed with it; these checks run before
# anything is handed to the library (shapes and dtypes first, then devices).

def _shape(t: torch.Tensor, shape, what: str):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _u8(t: torch.Tensor, shape, what: str):
    """A packed byte array: uint8, the given shape, contiguous (the ABI takes no row stride for it)."""
    if t.dtype != torch.uint8:
        raise TypeError(f"{what} must be uint8, got {t.dtype}")
    _shape(t, shape, what)
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")


def _f32_vec(t: torch.Tensor, n: int, what: str):
    if t.dtype != torch.float32 or t.numel() != n or not t.is_contiguous():
        raise ValueError(f"{what} must be a contiguous float32 tensor of {n} element(s), got {t.dtype} "
                         f"{tuple(t.shape)}")


def _matrix(t: torch.Tensor, shape, dtypes, what: str):
    if t.dtype not in dtypes:
        raise TypeError(f"{what} must be {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    _shape(t, shape, what)
    _ld(t)


def _out(out, M: int, N: int, dtype, like: torch.Tensor) -> torch.Tensor:
    """The GEMM / dequantize output: allocated when None, else checked (shape (M, N),
    float32 or bfloat16, unit stride along rows)."""
    if out is None:
        _out_dt(dtype)
        return torch.empty(M, N, dtype=dtype, device=like.device)
    _out_dt(out.dtype)
    _matrix(out, (M, N), (torch.float32, torch.bfloat16), "out")
    return out


def _workspace(ws, need: int, like: torch.Tensor) -> torch.Tensor:
    if ws is None:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=like.device)
    if ws.dtype != torch.uint8 or ws.dim() != 1 or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous 1-D uint8 tensor")
    if ws.numel() < need:
        raise ValueError(f"workspace holds {ws.numel()} bytes, {need} needed")
    return ws


def _k_match(K: int, cols: int):
    if K != cols:
        raise ValueError(f"A has K = {K} columns but the weight has {cols}")


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
    """The row stride (leading dimension) of a 2-D tensor with unit stride along its rows.
    A single row's stride is never followed, and torch may report any value for it
    (0 after unsqueeze or expand): it is given as the row length then."""
    if t.dim() != 2 or (t.stride(1) != 1 and t.shape[1] > 1):
        raise ValueError("expected a 2-D tensor with unit stride along its rows")
    if t.shape[0] <= 1:
        return max(t.stride(0), t.shape[1])
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

    def check(self, what="NVFP4 tensor"):
        _u8(self.codes, (self.rows, self.cols // 2), f"{what} codes")
        _u8(self.scales, (self.rows, self.cols // 16), f"{what} scales")
        _f32_vec(self.tscale, self.rows if self.per_row else 1, f"{what} tensor scale")
        return self


@dataclasses.dataclass
class PackedMXFP4:
    """MXFP4 tensor [rows, cols]: codes uint8 [rows, cols/2], scales uint8 [rows, cols/32] (E8M0)."""
    codes: torch.Tensor
    scales: torch.Tensor
    rows: int
    cols: int

    def nbytes(self) -> int:
        return self.codes.numel() + self.scales.numel()

    def check(self, what="MXFP4 tensor"):
        _u8(self.codes, (self.rows, self.cols // 2), f"{what} codes")
        _u8(self.scales, (self.rows, self.cols // 32), f"{what} scales")
        return self


# --------------------------------------------------------------- NVFP4 -----

def nvfp4_quantize(x: torch.Tensor, mode="tensor", nonfinite: torch.Tensor | None = None,
                   out: PackedNVFP4 | None = None, workspace: torch.Tensor | None = None) -> PackedNVFP4:
    """Quantize a 2-D fp32/bf16 device tensor to NVFP4 (blocks along its rows)."""
    L = lib()
    _dt(x)
    rows, cols = x.shape
    m = _mode(mode)
    if out is None:
        out = PackedNVFP4(torch.empty(rows, cols // 2, dtype=torch.uint8, device=x.device),
                          torch.empty(rows, cols // 16, dtype=torch.uint8, device=x.device),
                          torch.empty(rows if m == PER_ROW else 1, dtype=torch.float32, device=x.device),
                          rows, cols, m == PER_ROW)
    if (out.rows, out.cols, out.per_row) != (rows, cols, m == PER_ROW):
        raise ValueError("out does not describe this tensor and scale mode")
    out.check("out")
    if nonfinite is not None and (nonfinite.dtype != torch.int32 or nonfinite.numel() < 1):
        raise ValueError("nonfinite must be an int32 tensor of at least one element")
    wsb = L.nvfp4_quantize_workspace(rows, cols, m)
    workspace = _workspace(workspace, wsb, x) if wsb else workspace
    _need_cuda(x, nonfinite, out.codes, out.scales, out.tscale, workspace)
    _run(L.nvfp4_quantize, _ptr(x), _dt(x), rows, cols, _ld(x), _ptr(out.codes), _ptr(out.scales),
                            _ptr(out.tscale), m, _ptr(workspace), wsb, _ptr(nonfinite), _stream())
    return out


def nvfp4_dequantize(p: PackedNVFP4, dtype=torch.float32, out: torch.Tensor | None = None) -> torch.Tensor:
    L = lib()
    p.check("p")
    out = _out(out, p.rows, p.cols, dtype, p.codes)
    _need_cuda(p.codes, p.scales, p.tscale, out)
    _run(L.nvfp4_dequantize, _ptr(p.codes), _ptr(p.scales), _ptr(p.tscale),
                              PER_ROW if p.per_row else PER_TENSOR, p.rows, p.cols, _ptr(out),
                              _out_dt(out.dtype), _ld(out), _stream())
    return out


def _bf16_a(a: torch.Tensor, fn: str):
    if a.dtype != torch.bfloat16:
        raise TypeError(f"{fn} takes bfloat16 activations")
    if a.dim() != 2:
        raise ValueError(f"{fn} takes a 2-D activation tensor [M, K]")
    _ld(a)
    return a.shape


def _weight_nv(w: PackedNVFP4, K: int):
    if w.per_row:
        raise ValueError("NVFP4 weights carry one tensor scale (quantize them with mode='tensor')")
    w.check("w")
    _k_match(K, w.cols)


def gemm_w4a16(a: torch.Tensor, w: PackedNVFP4, dtype=torch.bfloat16,
               out: torch.Tensor | None = None) -> torch.Tensor:
    """C = A . W^T with bf16 A [M, K] and NVFP4 W [N, K] (per-tensor scale)."""
    L = lib()
    M, K = _bf16_a(a, "gemm_w4a16")
    _weight_nv(w, K)
    out = _out(out, M, w.rows, dtype, a)
    _need_cuda(a, w.codes, w.scales, w.tscale, out)
    _run(L.gemm_w4a16, _ptr(a), M, K, _ld(a), _ptr(w.codes), _ptr(w.scales), _ptr(w.tscale), w.rows,
                        _ptr(out), _out_dt(out.dtype), _ld(out), _stream())
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

    def check(self, what="w"):
        _u8(self.codes, (self.cols // 128, self.rows, 64), f"{what} codes")
        _u8(self.scales, (self.cols // 128, self.rows, 8), f"{what} scales")
        _f32_vec(self.tscale, 1, f"{what} tensor scale")
        return self


def nvfp4_pack_decode(w: PackedNVFP4, out: DecodeNVFP4 | None = None) -> DecodeNVFP4:
    """Rewrite a per-tensor NVFP4 weight into the decode layout (segment-major)."""
    L = lib()
    if w.per_row:
        raise ValueError("the decode layout holds weights with a per-tensor scale")
    w.check("w")
    N, K = w.rows, w.cols
    if out is None:
        dev = w.codes.device
        out = DecodeNVFP4(torch.empty(K // 128, N, 64, dtype=torch.uint8, device=dev),
                          torch.empty(K // 128, N, 8, dtype=torch.uint8, device=dev),
                          w.tscale, N, K)
    if (out.rows, out.cols) != (N, K):
        raise ValueError("out does not describe this weight")
    out.check("out")
    _need_cuda(w.codes, w.scales, out.codes, out.scales)
    _run(L.nvfp4_pack_decode, _ptr(w.codes), _ptr(w.scales), N, K, _ptr(out.codes), _ptr(out.scales),
                               _stream())
    return out


def read_ceiling(buf: torch.Tensor, grid: int, sink: torch.Tensor) -> None:
    """Measurement aid: read every byte of `buf` (a contiguous device tensor whose
    size is a multiple of 16 bytes) once, on `grid` workgroups, computing nothing
    from it.  `sink` is a device int32/uint32 tensor of at least one element."""
    L = lib()
    if not buf.is_contiguous() or buf.numel() * buf.element_size() % 16:
        raise ValueError("buf must be contiguous, a multiple of 16 bytes")
    if sink.dtype not in (torch.int32, torch.uint32) or sink.numel() < 1:
        raise ValueError("sink must hold one 32-bit integer")
    _need_cuda(buf, sink)
    _run(L.fp4blk_read_ceiling, _ptr(buf), buf.numel() * buf.element_size(), int(grid), _ptr(sink), _stream())


def gemm_w4a16_decode(a: torch.Tensor, w: DecodeNVFP4, dtype=torch.bfloat16,
                      out: torch.Tensor | None = None) -> torch.Tensor:
    """C = A . W^T for bf16 A [M, K] and W in the decode layout: the decode GEMV for M <= 16,
    the prefill GEMM on the same layout for larger M."""
    L = lib()
    M, K = _bf16_a(a, "gemm_w4a16_decode")
    w.check("w")
    _k_match(K, w.cols)
    out = _out(out, M, w.rows, dtype, a)
    _need_cuda(a, w.codes, w.scales, w.tscale, out)
    _run(L.gemm_w4a16_decode, _ptr(a), M, K, _ld(a), _ptr(w.codes), _ptr(w.scales), _ptr(w.tscale), w.rows,
                               _ptr(out), _out_dt(out.dtype), _ld(out), _stream())
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


def _w4a4(fn_name: str, a, w, a_mode, dtype, out, workspace, w_check):
    L = lib()
    M, K = _bf16_a(a, fn_name)
    w_check(w, K)
    m = _mode(a_mode)
    out = _out(out, M, w.rows, dtype, a)
    workspace = _workspace(workspace, L.gemm_w4a4_workspace(M, K, m), a)
    _need_cuda(a, w.codes, w.scales, w.tscale, out, workspace)
    _run(getattr(L, fn_name), _ptr(a), M, K, _ld(a), m, _ptr(w.codes), _ptr(w.scales), _ptr(w.tscale), w.rows,
                               _ptr(out), _out_dt(out.dtype), _ld(out), _ptr(workspace), workspace.numel(),
                               _stream())
    return out


def gemm_w4a4(a: torch.Tensor, w: PackedNVFP4, a_mode="row", dtype=torch.bfloat16,
              out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """NVFP4 W4A4: quantize bf16 A on the device (per row by default), then C = A_q . W^T."""
    return _w4a4("gemm_w4a4", a, w, a_mode, dtype, out, workspace, _weight_nv)


def gemm_w4a4_noalloc(a: torch.Tensor, w: PackedNVFP4, a_mode="row", dtype=torch.bfloat16,
                      out: torch.Tensor | None = None) -> torch.Tensor:
    """gemm_w4a4 with A's packed form in the library's own device scratch (32 MiB per
    device): the library allocates nothing.  Pass `out` to allocate nothing here either.
    Calls that overlap on one device race for the scratch."""
    L = lib()
    M, K = _bf16_a(a, "gemm_w4a4_noalloc")
    _weight_nv(w, K)
    m = _mode(a_mode)
    out = _out(out, M, w.rows, dtype, a)
    _need_cuda(a, w.codes, w.scales, w.tscale, out)
    _run(L.gemm_w4a4_noalloc, _ptr(a), M, K, _ld(a), m, _ptr(w.codes), _ptr(w.scales), _ptr(w.tscale), w.rows,
         _ptr(out), _out_dt(out.dtype), _ld(out), _stream())
    return out


def _prequant_nv(fn_name: str, a: PackedNVFP4, w, dtype, out):
    L = lib()
    a.check("a")
    _k_match(a.cols, w.cols)
    out = _out(out, a.rows, w.rows, dtype, a.codes)
    _need_cuda(a.codes, a.scales, a.tscale, w.codes, w.scales, w.tscale, out)
    _run(getattr(L, fn_name), _ptr(a.codes), _ptr(a.scales), _ptr(a.tscale),
                               PER_ROW if a.per_row else PER_TENSOR, a.rows, a.cols,
                               _ptr(w.codes), _ptr(w.scales), _ptr(w.tscale), w.rows, _ptr(out),
                               _out_dt(out.dtype), _ld(out), _stream())
    return out


def gemm_nvfp4_prequant(a: PackedNVFP4, w: PackedNVFP4, dtype=torch.bfloat16,
                        out: torch.Tensor | None = None) -> torch.Tensor:
    _weight_nv(w, a.cols)
    return _prequant_nv("gemm_nvfp4_w4a4_prequant", a, w, dtype, out)


def _weight_nv_dec(w: DecodeNVFP4, K: int):
    w.check("w")
    _k_match(K, w.cols)


def gemm_w4a4_seg(a: torch.Tensor, w: DecodeNVFP4, a_mode="row", dtype=torch.bfloat16,
                  out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """gemm_w4a4 with W in the decode layout: the same result."""
    return _w4a4("gemm_w4a4_seg", a, w, a_mode, dtype, out, workspace, _weight_nv_dec)


def gemm_nvfp4_prequant_seg(a: PackedNVFP4, w: DecodeNVFP4, dtype=torch.bfloat16,
                            out: torch.Tensor | None = None) -> torch.Tensor:
    """gemm_nvfp4_prequant with W in the decode layout."""
    _weight_nv_dec(w, a.cols)
    return _prequant_nv("gemm_nvfp4_w4a4_prequant_seg", a, w, dtype, out)


# --------------------------------------------------------------- MXFP4 -----

def mxfp4_quantize(x: torch.Tensor, rule="ocp", nonfinite: torch.Tensor | None = None,
                   out: PackedMXFP4 | None = None) -> PackedMXFP4:
    L = lib()
    _dt(x)
    rows, cols = x.shape
    if out is None:
        out = PackedMXFP4(torch.empty(rows, cols // 2, dtype=torch.uint8, device=x.device),
                          torch.empty(rows, cols // 32, dtype=torch.uint8, device=x.device), rows, cols)
    if (out.rows, out.cols) != (rows, cols):
        raise ValueError("out does not describe this tensor")
    out.check("out")
    if nonfinite is not None and (nonfinite.dtype != torch.int32 or nonfinite.numel() < 1):
        raise ValueError("nonfinite must be an int32 tensor of at least one element")
    _need_cuda(x, nonfinite, out.codes, out.scales)
    _run(L.mxfp4_quantize, _ptr(x), _dt(x), rows, cols, _ld(x), _ptr(out.codes), _ptr(out.scales),
                            _rule(rule), _ptr(nonfinite), _stream())
    return out


def mxfp4_dequantize(p: PackedMXFP4, dtype=torch.float32, out: torch.Tensor | None = None) -> torch.Tensor:
    L = lib()
    p.check("p")
    out = _out(out, p.rows, p.cols, dtype, p.codes)
    _need_cuda(p.codes, p.scales, out)
    _run(L.mxfp4_dequantize, _ptr(p.codes), _ptr(p.scales), p.rows, p.cols, _ptr(out),
                              _out_dt(out.dtype), _ld(out), _stream())
    return out


def _weight_mx(w: PackedMXFP4, K: int):
    w.check("w")
    _k_match(K, w.cols)


def _mx_full(fn_name: str, ws_name: str, a, w, rule, dtype, out, workspace, w_check):
    """The MXFP4 / W4A8 entry points that quantize bf16 A into a workspace first."""
    L = lib()
    M, K = _bf16_a(a, fn_name)
    w_check(w, K)
    r = _rule(rule)
    out = _out(out, M, w.rows, dtype, a)
    workspace = _workspace(workspace, getattr(L, ws_name)(M, K), a)
    _need_cuda(a, w.codes, w.scales, out, workspace)
    _run(getattr(L, fn_name), _ptr(a), M, K, _ld(a), r, _ptr(w.codes), _ptr(w.scales), w.rows,
                               _ptr(out), _out_dt(out.dtype), _ld(out), _ptr(workspace), workspace.numel(),
                               _stream())
    return out


def _mx_prequant(fn_name: str, a, w, dtype, out):
    L = lib()
    a.check("a")
    _k_match(a.cols, w.cols)
    out = _out(out, a.rows, w.rows, dtype, a.codes)
    _need_cuda(a.codes, a.scales, w.codes, w.scales, out)
    _run(getattr(L, fn_name), _ptr(a.codes), _ptr(a.scales), a.rows, a.cols, _ptr(w.codes), _ptr(w.scales),
                               w.rows, _ptr(out), _out_dt(out.dtype), _ld(out), _stream())
    return out


def mxfp4_gemm_w4a4(a: torch.Tensor, w: PackedMXFP4, rule="ocp", dtype=torch.bfloat16,
                    out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    return _mx_full("mxfp4_gemm_w4a4", "mxfp4_gemm_w4a4_workspace", a, w, rule, dtype, out, workspace, _weight_mx)


def mxfp4_packed_a(ws: torch.Tensor, M: int, K: int, N: int):
    """Views of A's MXFP4 form inside the workspace of an mxfp4_gemm_w4a4 call
    with W of N rows: segment-major (DecodeMXFP4) or row-major (PackedMXFP4), as
    the library reports for those sizes."""
    if lib().mxfp4_gemm_w4a4_a_segment_major(M, N, K):
        return mxfp4_seg_packed_a(ws, M, K)
    cb = (M * (K // 2) + 255) // 256 * 256
    return PackedMXFP4(ws[:M * K // 2].view(M, K // 2), ws[cb:cb + M * K // 32].view(M, K // 32), M, K)


def mxfp4_gemm_prequant(a: PackedMXFP4, w: PackedMXFP4, dtype=torch.bfloat16,
                        out: torch.Tensor | None = None) -> torch.Tensor:
    w.check("w")
    return _mx_prequant("mxfp4_gemm_prequant", a, w, dtype, out)


def mxfp4_gemm_w4a16(a: torch.Tensor, w: PackedMXFP4, dtype=torch.bfloat16,
                     out: torch.Tensor | None = None) -> torch.Tensor:
    """C = A . W^T with bf16 A [M, K] and MXFP4 W [N, K] (K % 128 == 0)."""
    L = lib()
    M, K = _bf16_a(a, "mxfp4_gemm_w4a16")
    _weight_mx(w, K)
    out = _out(out, M, w.rows, dtype, a)
    _need_cuda(a, w.codes, w.scales, out)
    _run(L.mxfp4_gemm_w4a16, _ptr(a), M, K, _ld(a), _ptr(w.codes), _ptr(w.scales), w.rows,
                              _ptr(out), _out_dt(out.dtype), _ld(out), _stream())
    return out


@dataclasses.dataclass
class DecodeMXFP4:
    """An MXFP4 weight [rows, cols] in the decode layout (see mxfp4_pack_decode):
    codes [cols/128, rows, 64], scales [cols/128, rows, 4]."""
    codes: torch.Tensor
    scales: torch.Tensor
    rows: int
    cols: int

    def check(self, what="w"):
        _u8(self.codes, (self.cols // 128, self.rows, 64), f"{what} codes")
        _u8(self.scales, (self.cols // 128, self.rows, 4), f"{what} scales")
        return self


def _weight_mx_dec(w: DecodeMXFP4, K: int):
    w.check("w")
    _k_match(K, w.cols)


def mxfp4_pack_decode(w: PackedMXFP4, out: DecodeMXFP4 | None = None) -> DecodeMXFP4:
    """Rewrite an MXFP4 weight into the decode layout (segment-major)."""
    L = lib()
    w.check("w")
    N, K = w.rows, w.cols
    if out is None:
        dev = w.codes.device
        out = DecodeMXFP4(torch.empty(K // 128, N, 64, dtype=torch.uint8, device=dev),
                          torch.empty(K // 128, N, 4, dtype=torch.uint8, device=dev), N, K)
    if (out.rows, out.cols) != (N, K):
        raise ValueError("out does not describe this weight")
    out.check("out")
    _need_cuda(w.codes, w.scales, out.codes, out.scales)
    _run(L.mxfp4_pack_decode, _ptr(w.codes), _ptr(w.scales), N, K, _ptr(out.codes), _ptr(out.scales),
                               _stream())
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
    return _mx_full("mxfp4_gemm_w4a4_seg", "mxfp4_gemm_w4a4_seg_workspace", a, w, rule, dtype, out, workspace,
                    _weight_mx_dec)


def mxfp4_gemm_prequant_seg(a: DecodeMXFP4, w: DecodeMXFP4, dtype=torch.bfloat16,
                            out: torch.Tensor | None = None) -> torch.Tensor:
    """The GEMM half of mxfp4_gemm_w4a4_seg: A and W both in the segment-major layout."""
    w.check("w")
    return _mx_prequant("mxfp4_gemm_prequant_seg", a, w, dtype, out)


def mxfp4_gemm_w4a16_decode(a: torch.Tensor, w: DecodeMXFP4, dtype=torch.bfloat16,
                            out: torch.Tensor | None = None) -> torch.Tensor:
    """C = A . W^T for bf16 A [M, K] and an MXFP4 W in the decode layout (GEMV for M <= 16,
    the prefill GEMM on the same layout for larger M)."""
    L = lib()
    M, K = _bf16_a(a, "mxfp4_gemm_w4a16_decode")
    _weight_mx_dec(w, K)
    out = _out(out, M, w.rows, dtype, a)
    _need_cuda(a, w.codes, w.scales, out)
    _run(L.mxfp4_gemm_w4a16_decode, _ptr(a), M, K, _ld(a), _ptr(w.codes), _ptr(w.scales), w.rows,
                                     _ptr(out), _out_dt(out.dtype), _ld(out), _stream())
    return out


@dataclasses.dataclass
class PackedMXFP8:
    """An MXFP8 tensor [rows, cols]: E4M3FN codes [rows, cols], E8M0 scales [rows, cols/32]."""
    codes: torch.Tensor
    scales: torch.Tensor
    rows: int
    cols: int

    def check(self, what="MXFP8 tensor"):
        _u8(self.codes, (self.rows, self.cols), f"{what} codes")
        _u8(self.scales, (self.rows, self.cols // 32), f"{what} scales")
        return self


def mxfp8_quantize(x: torch.Tensor, rule="ocp", nonfinite: torch.Tensor | None = None,
                   out: PackedMXFP8 | None = None) -> PackedMXFP8:
    """MXFP8 (E4M3FN elements, E8M0 per 32) of an fp32 or bf16 [rows, cols] tensor."""
    L = lib()
    _dt(x)
    rows, cols = x.shape
    if out is None:
        out = PackedMXFP8(torch.empty(rows, cols, dtype=torch.uint8, device=x.device),
                          torch.empty(rows, cols // 32, dtype=torch.uint8, device=x.device), rows, cols)
    if (out.rows, out.cols) != (rows, cols):
        raise ValueError("out does not describe this tensor")
    out.check("out")
    if nonfinite is not None and (nonfinite.dtype != torch.int32 or nonfinite.numel() < 1):
        raise ValueError("nonfinite must be an int32 tensor of at least one element")
    _need_cuda(x, nonfinite, out.codes, out.scales)
    _run(L.mxfp8_quantize, _ptr(x), _dt(x), rows, cols, _ld(x), _ptr(out.codes), _ptr(out.scales),
                            _rule(rule), _ptr(nonfinite), _stream())
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
    return _mx_full("mxfp4_gemm_w4a8", "mxfp4_gemm_w4a8_workspace", a, w, rule, dtype, out, workspace, _weight_mx)


def mxfp4_gemm_w4a8_prequant(a: PackedMXFP8, w: PackedMXFP4, dtype=torch.bfloat16,
                             out: torch.Tensor | None = None) -> torch.Tensor:
    """The GEMM half of mxfp4_gemm_w4a8 on an MXFP8 A."""
    w.check("w")
    return _mx_prequant("mxfp4_gemm_w4a8_prequant", a, w, dtype, out)


def mxfp4_gemm_w4a8_seg(a: torch.Tensor, w: DecodeMXFP4, rule="ocp", dtype=torch.bfloat16,
                        out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """W4A8 with the MXFP4 W in the decode (segment-major) layout; the same result as mxfp4_gemm_w4a8."""
    return _mx_full("mxfp4_gemm_w4a8_seg", "mxfp4_gemm_w4a8_workspace", a, w, rule, dtype, out, workspace,
                    _weight_mx_dec)


def mxfp4_gemm_w4a8_prequant_seg(a: PackedMXFP8, w: DecodeMXFP4, dtype=torch.bfloat16,
                                 out: torch.Tensor | None = None) -> torch.Tensor:
    """The GEMM half of mxfp4_gemm_w4a8_seg on an MXFP8 A."""
    w.check("w")
    return _mx_prequant("mxfp4_gemm_w4a8_prequant_seg", a, w, dtype, out)


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

    def check(self, what="w"):
        _u8(self.codes, (self.experts, self.rows, self.cols // 2), f"{what} codes")
        _u8(self.scales, (self.experts, self.rows, self.cols // 16), f"{what} scales")
        _f32_vec(self.tscale, self.experts, f"{what} tensor scales")
        return self


@dataclasses.dataclass
class ExpertsMXFP4:
    """E MXFP4 expert weights [E, N, K]: codes uint8 [E, N, K/2], scales uint8 [E, N, K/32]."""
    codes: torch.Tensor
    scales: torch.Tensor
    experts: int
    rows: int
    cols: int

    def check(self, what="w"):
        _u8(self.codes, (self.experts, self.rows, self.cols // 2), f"{what} codes")
        _u8(self.scales, (self.experts, self.rows, self.cols // 32), f"{what} scales")
        return self


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


def _grouped_common(a_rows, K, w, group_offs, row_index):
    """Checks the grouping and the experts; returns (grouped rows, groups)."""
    if group_offs.dtype != torch.int32 or group_offs.dim() != 1 or not group_offs.is_contiguous():
        raise TypeError("group_offs must be a contiguous 1-D int32 device tensor [groups + 1]")
    if row_index is not None and (row_index.dtype != torch.int32 or row_index.dim() != 1
                                  or not row_index.is_contiguous()):
        raise TypeError("row_index must be a contiguous 1-D int32 device tensor [rows]")
    groups = group_offs.numel() - 1
    if groups != w.experts:
        raise ValueError(f"group_offs describes {groups} groups but the weight holds {w.experts} experts")
    w.check("w")
    _k_match(K, w.cols)
    rows = row_index.numel() if row_index is not None else a_rows
    return rows, groups


def nvfp4_grouped_gemm_w4a16(a: torch.Tensor, w: ExpertsNVFP4, group_offs: torch.Tensor,
                             row_index: torch.Tensor | None = None, dtype=torch.bfloat16,
                             out: torch.Tensor | None = None) -> torch.Tensor:
    """C[t] = A[row_index[t]] . W_e^T for the grouped rows t of group e (bf16 A, NVFP4 experts)."""
    L = lib()
    a_rows, K = _bf16_a(a, "nvfp4_grouped_gemm_w4a16")
    rows, groups = _grouped_common(a_rows, K, w, group_offs, row_index)
    out = _out(out, rows, w.rows, dtype, a)
    _need_cuda(a, w.codes, w.scales, w.tscale, group_offs, row_index, out)
    _run(L.nvfp4_grouped_gemm_w4a16, _ptr(a), a_rows, K, _ld(a), _ptr(row_index), _ptr(group_offs),
                                      groups, rows, _ptr(w.codes), _ptr(w.scales), _ptr(w.tscale), w.rows,
                                      _ptr(out), _out_dt(out.dtype), _ld(out), _stream())
    return out


def mxfp4_grouped_gemm_w4a16(a: torch.Tensor, w: ExpertsMXFP4, group_offs: torch.Tensor,
                             row_index: torch.Tensor | None = None, dtype=torch.bfloat16,
                             out: torch.Tensor | None = None) -> torch.Tensor:
    """As nvfp4_grouped_gemm_w4a16 with MXFP4 experts."""
    L = lib()
    a_rows, K = _bf16_a(a, "mxfp4_grouped_gemm_w4a16")
    rows, groups = _grouped_common(a_rows, K, w, group_offs, row_index)
    out = _out(out, rows, w.rows, dtype, a)
    _need_cuda(a, w.codes, w.scales, group_offs, row_index, out)
    _run(L.mxfp4_grouped_gemm_w4a16, _ptr(a), a_rows, K, _ld(a), _ptr(row_index), _ptr(group_offs),
                                      groups, rows, _ptr(w.codes), _ptr(w.scales), w.rows, _ptr(out),
                                      _out_dt(out.dtype), _ld(out), _stream())
    return out


def nvfp4_grouped_gemm_w4a4_workspace(a_rows: int, K: int, device="cuda") -> torch.Tensor:
    return torch.empty(lib().nvfp4_grouped_gemm_w4a4_workspace(a_rows, K), dtype=torch.uint8, device=device)


def nvfp4_grouped_gemm_w4a4(a: torch.Tensor, w: ExpertsNVFP4, group_offs: torch.Tensor,
                            row_index: torch.Tensor | None = None, dtype=torch.bfloat16,
                            out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """NVFP4 W4A4 grouped GEMM: every A row quantized once per row, then gathered per group."""
    L = lib()
    a_rows, K = _bf16_a(a, "nvfp4_grouped_gemm_w4a4")
    rows, groups = _grouped_common(a_rows, K, w, group_offs, row_index)
    out = _out(out, rows, w.rows, dtype, a)
    workspace = _workspace(workspace, L.nvfp4_grouped_gemm_w4a4_workspace(a_rows, K), a)
    _need_cuda(a, w.codes, w.scales, w.tscale, group_offs, row_index, out, workspace)
    _run(L.nvfp4_grouped_gemm_w4a4, _ptr(a), a_rows, K, _ld(a), _ptr(row_index), _ptr(group_offs),
                                     groups, rows, _ptr(w.codes), _ptr(w.scales), _ptr(w.tscale), w.rows,
                                     _ptr(out), _out_dt(out.dtype), _ld(out), _ptr(workspace), workspace.numel(),
                                     _stream())
    return out


def nvfp4_grouped_gemm_w4a4_prequant(a: PackedNVFP4, w: ExpertsNVFP4, group_offs: torch.Tensor,
                                     row_index: torch.Tensor | None = None, dtype=torch.bfloat16,
                                     out: torch.Tensor | None = None) -> torch.Tensor:
    """The GEMM half of nvfp4_grouped_gemm_w4a4 on a per-row NVFP4 A."""
    L = lib()
    if not a.per_row:
        raise ValueError("the grouped W4A4 GEMM takes a per-row NVFP4 A")
    a.check("a")
    rows, groups = _grouped_common(a.rows, a.cols, w, group_offs, row_index)
    out = _out(out, rows, w.rows, dtype, a.codes)
    _need_cuda(a.codes, a.scales, a.tscale, w.codes, w.scales, w.tscale, group_offs, row_index, out)
    _run(L.nvfp4_grouped_gemm_w4a4_prequant, _ptr(a.codes), _ptr(a.scales), _ptr(a.tscale), a.rows, a.cols,
                                              _ptr(row_index), _ptr(group_offs), groups, rows, _ptr(w.codes),
                                              _ptr(w.scales), _ptr(w.tscale), w.rows, _ptr(out),
                                              _out_dt(out.dtype), _ld(out), _stream())
    return out
