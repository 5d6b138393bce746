"""CPU oracle for NVFP4 / MXFP4 block-scaled quantization and the GEMMs it feeds.

TEST INFRASTRUCTURE.  Only ``tests/``, the smoke check and the benchmark's CPU
baseline leg may import this package.  The product path (the HIP library and
its Python binding) never imports it, and it imports nothing from them: the two
share only the seeded inputs of the ``synthetic`` module.

The arithmetic lives in ``fp4_oracle.c`` (plain scalar C, built with gcc, no
fast-math, no FP contraction); this module marshals numpy arrays to it and adds
the fp64 GEMM reference (numpy's float64 matmul over the exactly dequantized
operands, for shapes where the C triple loop would be slow).

Definitions followed (cited by page title and section):

* "NVFP4" (newton.com.tw wiki), "Technical principle": E2M1 elements, 16-value
  micro-blocks with an E4M3 scale each, one FP32 per-tensor scale, ~4.5 bits/value.
* Edge-FP4 article (eefocus.com), "FP4 as the next core standard": MXFP4 with
  32-element blocks sharing one E8M0 scale, 4.25 bits/weight.
* Unsloth Dynamic NVFP4 article (aixq.cc), "Core difference: W4A4 vs W4A16":
  W4A16 = dequantized 4-bit weights times 16-bit activations; W4A4 quantizes the
  activations as well.

Pins: every function here is checked by ``tests/test_oracle_*.py`` against
enumerations, library codecs (torch's float8 / bfloat16 casts), closed forms,
exact round trips and brute force; see those files.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp4_oracle.c")
_LIB = os.path.join(_HERE, "libfp4oracle.so")

F32, BF16 = 0, 1
PER_TENSOR, PER_ROW = 0, 1
MX_OCP_FLOOR, MX_CEIL = 0, 1
TENSOR_SCALE_DIVISOR = 2688.0  # 6 (largest E2M1) * 448 (largest E4M3)


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C, OpenMP over rows, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", "-fexcess-precision=standard", "-Wall", "-Wextra",
               _SRC, "-o", _LIB + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        L.fp4o_e2m1_decode.restype = ctypes.c_double
        L.fp4o_e2m1_decode.argtypes = [ctypes.c_uint8]
        L.fp4o_e2m1_encode.restype = ctypes.c_uint8
        L.fp4o_e2m1_encode.argtypes = [ctypes.c_double]
        L.fp4o_e4m3_decode.restype = ctypes.c_double
        L.fp4o_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.fp4o_e4m3_encode_sat.restype = ctypes.c_uint8
        L.fp4o_e4m3_encode_sat.argtypes = [ctypes.c_float]
        L.fp4o_e8m0_decode.restype = ctypes.c_double
        L.fp4o_e8m0_decode.argtypes = [ctypes.c_uint8]
        L.fp4o_e2m1_encode_f32.argtypes = [p, i64, p]
        L.fp4o_e4m3_encode_f32.argtypes = [p, i64, p]
        L.fp4o_f32_to_bf16_n.argtypes = [p, i64, p]
        L.fp4o_nvfp4_quantize.restype = ctypes.c_int
        L.fp4o_nvfp4_quantize.argtypes = [p, ctypes.c_int, i64, i64, i64, p, p, p, ctypes.c_int]
        L.fp4o_nvfp4_dequantize.argtypes = [p, p, p, ctypes.c_int, i64, i64, p]
        L.fp4o_nvfp4_to_f64.argtypes = [p, p, p, ctypes.c_int, i64, i64, p]
        L.fp4o_mxfp4_quantize.argtypes = [p, ctypes.c_int, i64, i64, i64, p, p, ctypes.c_int]
        L.fp4o_mxfp4_dequantize.argtypes = [p, p, i64, i64, p]
        L.fp4o_mxfp4_to_f64.argtypes = [p, p, i64, i64, p]
        L.fp4o_mxfp8_quantize.argtypes = [p, ctypes.c_int, i64, i64, i64, p, p, ctypes.c_int]
        L.fp4o_mxfp8_to_f64.argtypes = [p, p, i64, i64, p]
        L.fp4o_int4_quantize.argtypes = [p, ctypes.c_int, i64, i64, i64, ctypes.c_int, ctypes.c_int, p, p, p]
        L.fp4o_gemm_f64.argtypes = [p, p, i64, i64, i64, p, p]
        L.fp4o_num_threads.restype = ctypes.c_int
        L.fp4o_num_threads.argtypes = []
        _lib = L
    return _lib


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(lib().fp4o_num_threads())


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _input(x: np.ndarray):
    """fp32 array, or bfloat16 given as uint16 bit patterns."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, F32
    if x.dtype == np.uint16:
        return x, BF16
    raise TypeError(f"oracle input must be float32 or bf16 bits (uint16), got {x.dtype}")


# ------------------------------------------------------------------ codecs --

def e2m1_decode(c: int) -> float:
    return lib().fp4o_e2m1_decode(int(c))


def e2m1_encode(v: float) -> int:
    return lib().fp4o_e2m1_encode(float(v))


def e4m3_decode(b: int) -> float:
    return lib().fp4o_e4m3_decode(int(b))


def e4m3_encode_sat(q: float) -> int:
    return lib().fp4o_e4m3_encode_sat(float(q))


def e8m0_decode(b: int) -> float:
    return lib().fp4o_e8m0_decode(int(b))


def e2m1_encode_array(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().fp4o_e2m1_encode_f32(_ptr(v), v.size, _ptr(out))
    return out


def e4m3_encode_array(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().fp4o_e4m3_encode_f32(_ptr(v), v.size, _ptr(out))
    return out


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, np.uint16)
    lib().fp4o_f32_to_bf16_n(_ptr(v), v.size, _ptr(out))
    return out


# ------------------------------------------------------------------- NVFP4 --

def nvfp4_quantize(x: np.ndarray, per_row: bool = False):
    """x: [rows, cols] fp32 or bf16 bits, cols % 16 == 0.

    Returns (codes uint8 [rows, cols/2], scales uint8 [rows, cols/16],
    tscale float32 [1] or [rows])."""
    x, dt = _input(x)
    rows, cols = x.shape
    if cols % 16:
        raise ValueError("NVFP4 needs whole 16-element blocks along the last axis")
    codes = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows, cols // 16), np.uint8)
    tscale = np.empty(rows if per_row else 1, np.float32)
    lib().fp4o_nvfp4_quantize(_ptr(x), dt, rows, cols, cols, _ptr(codes), _ptr(scales),
                              _ptr(tscale), int(per_row))
    return codes, scales, tscale


def nvfp4_dequantize(codes, scales, tscale, per_row: bool = False) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    tscale = np.ascontiguousarray(tscale, np.float32)
    rows, cols = codes.shape[0], codes.shape[1] * 2
    y = np.empty((rows, cols), np.float32)
    lib().fp4o_nvfp4_dequantize(_ptr(codes), _ptr(scales), _ptr(tscale), int(per_row), rows,
                                cols, _ptr(y))
    return y


def nvfp4_to_f64(codes, scales, tscale, per_row: bool = False) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    tscale = np.ascontiguousarray(tscale, np.float32)
    rows, cols = codes.shape[0], codes.shape[1] * 2
    y = np.empty((rows, cols), np.float64)
    lib().fp4o_nvfp4_to_f64(_ptr(codes), _ptr(scales), _ptr(tscale), int(per_row), rows, cols,
                            _ptr(y))
    return y


# ------------------------------------------------------------------- MXFP4 --

def mxfp4_quantize(x: np.ndarray, rule: int = MX_OCP_FLOOR):
    """x: [rows, cols] fp32 or bf16 bits, cols % 32 == 0.

    Returns (codes uint8 [rows, cols/2], scales uint8 [rows, cols/32] E8M0)."""
    x, dt = _input(x)
    rows, cols = x.shape
    if cols % 32:
        raise ValueError("MXFP4 needs whole 32-element blocks along the last axis")
    codes = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows, cols // 32), np.uint8)
    lib().fp4o_mxfp4_quantize(_ptr(x), dt, rows, cols, cols, _ptr(codes), _ptr(scales), int(rule))
    return codes, scales


def mxfp4_dequantize(codes, scales) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    rows, cols = codes.shape[0], codes.shape[1] * 2
    y = np.empty((rows, cols), np.float32)
    lib().fp4o_mxfp4_dequantize(_ptr(codes), _ptr(scales), rows, cols, _ptr(y))
    return y


def mxfp4_to_f64(codes, scales) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    rows, cols = codes.shape[0], codes.shape[1] * 2
    y = np.empty((rows, cols), np.float64)
    lib().fp4o_mxfp4_to_f64(_ptr(codes), _ptr(scales), rows, cols, _ptr(y))
    return y


def mxfp8_quantize(x: np.ndarray, rule: int = MX_OCP_FLOOR):
    """MXFP8 (E4M3FN elements, E8M0 per 32): x [rows, cols] fp32 or bf16 bits,
    cols % 32 == 0.  Returns (codes uint8 [rows, cols], scales uint8 [rows, cols/32])."""
    x, dt = _input(x)
    rows, cols = x.shape
    if cols % 32:
        raise ValueError("MXFP8 needs whole 32-element blocks along the last axis")
    codes = np.empty((rows, cols), np.uint8)
    scales = np.empty((rows, cols // 32), np.uint8)
    lib().fp4o_mxfp8_quantize(_ptr(x), dt, rows, cols, cols, _ptr(codes), _ptr(scales), int(rule))
    return codes, scales


def mxfp8_to_f64(codes, scales) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    rows, cols = codes.shape
    y = np.empty((rows, cols), np.float64)
    lib().fp4o_mxfp8_to_f64(_ptr(codes), _ptr(scales), rows, cols, _ptr(y))
    return y


# -------------------------------------------------------------------- INT4 --
#
# The integer baseline (edge-FP4 article, section on why FP4 suits compression;
# NVFP4 wiki, competition section).  Symmetric levels -7..7, one step per block;
# the step's container is one of the INT4_* kinds (see fp4o_int4_quantize).

INT4_F32, INT4_BF16, INT4_E4M3_TENSOR, INT4_E8M0 = 0, 1, 2, 3


def int4_quantize(x: np.ndarray, block: int, kind: int):
    """x [rows, cols] fp32 or bf16 bits, cols % block == 0.  Returns (codes int8
    [rows, cols], step float64 [rows, cols / block], tensor scale float32 (kind 2))."""
    x, dt = _input(x)
    rows, cols = x.shape
    if cols % block:
        raise ValueError("INT4 needs whole blocks along the last axis")
    codes = np.empty((rows, cols), np.int8)
    step = np.empty((rows, cols // block), np.float64)
    ts = np.zeros(1, np.float32)
    lib().fp4o_int4_quantize(_ptr(x), dt, rows, cols, cols, int(block), int(kind), _ptr(codes), _ptr(step), _ptr(ts))
    return codes, step, ts[0]


def int4_to_f64(codes, step) -> np.ndarray:
    """codes x step, exactly, in fp64."""
    block = codes.shape[1] // step.shape[1]
    return codes.astype(np.float64) * np.repeat(np.asarray(step, np.float64), block, axis=1)


# -------------------------------------------------------------------- GEMM --

def gemm_f64_loop(a: np.ndarray, w: np.ndarray):
    """C = a @ w.T and T = |a| @ |w|.T by a plain fp64 triple loop (C)."""
    a = np.ascontiguousarray(a, np.float64)
    w = np.ascontiguousarray(w, np.float64)
    M, K = a.shape
    N = w.shape[0]
    c = np.empty((M, N), np.float64)
    t = np.empty((M, N), np.float64)
    lib().fp4o_gemm_f64(_ptr(a), _ptr(w), M, N, K, _ptr(c), _ptr(t))
    return c, t


def gemm_f64(a: np.ndarray, w: np.ndarray):
    """Same as gemm_f64_loop via numpy's float64 matmul (a library primitive)."""
    a = np.asarray(a, np.float64)
    w = np.asarray(w, np.float64)
    return a @ w.T, np.abs(a) @ np.abs(w).T


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def gemm_w4a16_ref(a_bf16: np.ndarray, w_codes, w_scales, w_tscale, rows=None):
    """fp64 reference of C = A . W^T with W dequantized exactly (NVFP4, per tensor).

    ``rows`` (optional index array) restricts the reference to those rows of A.
    Returns (C_ref, T) with T = sum_k |a w| (tolerance scale)."""
    a = bf16_bits_to_f64(a_bf16 if rows is None else a_bf16[rows])
    w = nvfp4_to_f64(w_codes, w_scales, w_tscale, per_row=False)
    return gemm_f64(a, w)


def gemm_w4a4_ref(a_bf16: np.ndarray, w_codes, w_scales, w_tscale, a_per_row=True, rows=None):
    """fp64 reference of the NVFP4 W4A4 GEMM: A quantized (per row by default) by
    this oracle, both operands dequantized exactly, then an fp64 product."""
    ac, asc, ats = nvfp4_quantize(a_bf16, per_row=a_per_row)
    if rows is not None:
        ac, asc = ac[rows], asc[rows]
        ats = ats[rows] if a_per_row else ats
    a = nvfp4_to_f64(ac, asc, ats, per_row=a_per_row)
    w = nvfp4_to_f64(w_codes, w_scales, w_tscale, per_row=False)
    return gemm_f64(a, w)


def mxfp4_gemm_w4a16_ref(a_bf16: np.ndarray, w_codes, w_scales, rows=None):
    """fp64 reference of C = A . W^T with bf16 A and W dequantized exactly (MXFP4:
    E2M1 times the block's E8M0 power of two; no tensor scale).  Returns (C_ref, T)."""
    a = bf16_bits_to_f64(a_bf16 if rows is None else a_bf16[rows])
    w = mxfp4_to_f64(w_codes, w_scales)
    return gemm_f64(a, w)


def mxfp4_gemm_w4a8_ref(a_bf16: np.ndarray, w_codes, w_scales, rule=MX_OCP_FLOOR, rows=None):
    """fp64 reference of the W4A8 GEMM: A quantized to MXFP8 by this oracle, W
    MXFP4, both dequantized exactly, then an fp64 product.  Returns (C_ref, T)."""
    src = a_bf16 if rows is None else a_bf16[rows]
    ac, asc = mxfp8_quantize(src, rule)
    a = mxfp8_to_f64(ac, asc)
    w = mxfp4_to_f64(w_codes, w_scales)
    return gemm_f64(a, w)


def mxfp4_gemm_w4a4_ref(a_bf16: np.ndarray, w_codes, w_scales, rule=MX_OCP_FLOOR, rows=None):
    """fp64 reference of the MXFP4 W4A4 GEMM (A quantized by this oracle)."""
    src = a_bf16 if rows is None else a_bf16[rows]
    ac, asc = mxfp4_quantize(src, rule)
    a = mxfp4_to_f64(ac, asc)
    w = mxfp4_to_f64(w_codes, w_scales)
    return gemm_f64(a, w)


# ------------------------------------------------------- grouped (MoE) --
#
# Mixture-of-experts layers (edge-FP4 article, eefocus.com, "FP4 as the next core
# standard": expert weights in MXFP4; Unsloth Dynamic NVFP4 article, aixq.cc,
# throughput section: a mixture-of-experts model with NVFP4 weights, W4A16 and
# all-W4A4).  Grouped row t of group e (group_offs[e] <= t < group_offs[e + 1])
# is C[t] = A[row_index[t]] . W_e^T, over exactly dequantized operands in fp64.

def _grouped_ref(a_f64, w_f64_of, group_offs, row_index, rows):
    offs = np.asarray(group_offs, np.int64)
    sel = np.arange(int(offs[-1])) if rows is None else np.asarray(rows, np.int64)
    grp = np.searchsorted(offs, sel, side="right") - 1     # last group starting at or before t
    arow = sel if row_index is None else np.asarray(row_index, np.int64)[sel]
    out_c = out_t = None
    for e in np.unique(grp):
        m = grp == e
        c, t = gemm_f64(a_f64[arow[m]], w_f64_of(int(e)))
        if out_c is None:
            out_c = np.zeros((len(sel), c.shape[1]))
            out_t = np.zeros((len(sel), c.shape[1]))
        out_c[m], out_t[m] = c, t
    return out_c, out_t


def nvfp4_grouped_gemm_w4a16_ref(a_bf16, w_codes, w_scales, w_tscale, group_offs, row_index=None, rows=None):
    """fp64 grouped W4A16 with NVFP4 experts (codes [E, N, K/2], scales [E, N, K/16],
    tensor scales [E]); ``rows`` restricts it to those grouped rows.  Returns (C_ref, T)."""
    a = bf16_bits_to_f64(a_bf16)
    return _grouped_ref(a, lambda e: nvfp4_to_f64(w_codes[e], w_scales[e], np.asarray(w_tscale)[e:e + 1]),
                        group_offs, row_index, rows)


def mxfp4_grouped_gemm_w4a16_ref(a_bf16, w_codes, w_scales, group_offs, row_index=None, rows=None):
    """fp64 grouped W4A16 with MXFP4 experts (codes [E, N, K/2], scales [E, N, K/32])."""
    a = bf16_bits_to_f64(a_bf16)
    return _grouped_ref(a, lambda e: mxfp4_to_f64(w_codes[e], w_scales[e]), group_offs, row_index, rows)


def nvfp4_grouped_gemm_w4a4_ref(a_bf16, w_codes, w_scales, w_tscale, group_offs, row_index=None, rows=None):
    """fp64 grouped NVFP4 W4A4: every A row quantized per row by this oracle, then
    dequantized exactly, gathered per group and multiplied by the expert."""
    ac, asc, ats = nvfp4_quantize(a_bf16, per_row=True)
    a = nvfp4_to_f64(ac, asc, ats, per_row=True)
    return _grouped_ref(a, lambda e: nvfp4_to_f64(w_codes[e], w_scales[e], np.asarray(w_tscale)[e:e + 1]),
                        group_offs, row_index, rows)
