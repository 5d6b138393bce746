"""Quantization-error study: NVFP4 vs MXFP4 (both scale rules) vs INT4.

TEST INFRASTRUCTURE (part of the oracle; CPU only).  It measures, on seeded
bell-shaped and heavy-tailed tensors, what the pages claim qualitatively:

* "NVFP4" (newton.com.tw wiki), "Technical principle": 16-value blocks with a
  fractional E4M3 scale fit local dynamic range better than MXFP4's 32-value
  blocks, and so quantize with less error.
* Edge-FP4 article (eefocus.com), section on why FP4 suits compression: INT4's
  evenly spaced levels lack a floating-point dynamic range, while E2M1's levels
  are dense near zero and sparse far from it, which suits bell-shaped data and
  keeps outliers; NVFP4 wiki, competition section: INT4 versions lose more
  accuracy than FP4 on some tasks.

INT4 has no fixed layout on the pages; it is measured in four containers (see
fp4o_int4_quantize): NVFP4's (16-blocks, E4M3 step and fp32 tensor scale),
MXFP4's (32-blocks, power-of-two step), and two common in practice (128-groups
with a bf16 step, one fp32 step per row).

Metrics per (distribution, format): SQNR = 10 log10(|x|^2 / |x - q(x)|^2) over
the whole tensor; the same over the elements at or below the median |x| (how
small values survive next to large ones); and the relative Frobenius error of a
W4A16 product A . q(W)^T with bf16 activations (the workload's recipe) against
the unquantized product.

    python -m oracle.error_study [--rows R --cols C]    prints the markdown table
"""
from __future__ import annotations

import argparse

import numpy as np

from . import (INT4_BF16, INT4_E4M3_TENSOR, INT4_E8M0, INT4_F32, MX_CEIL, MX_OCP_FLOOR, bf16_bits_to_f64,
               int4_quantize, int4_to_f64, mxfp4_quantize, mxfp4_to_f64, nvfp4_quantize, nvfp4_to_f64)

DISTRIBUTIONS = ["gaussian", "gaussian_outliers", "student_t3", "laplace", "channel_outliers"]


def _formats(cols):
    """name -> (bits per value, x [rows, cols] fp32 -> fp64 reconstruction)."""
    def nv(x):
        c, s, t = nvfp4_quantize(x)
        return nvfp4_to_f64(c, s, t)

    def mx(rule):
        def f(x):
            c, s = mxfp4_quantize(x, rule)
            return mxfp4_to_f64(c, s)
        return f

    def i4(block, kind):
        def f(x):
            c, d, _ = int4_quantize(x, block, kind)
            return int4_to_f64(c, d)
        return f

    return {
        "NVFP4 (16, E4M3 + fp32)": (4.5, nv),
        "MXFP4 OCP floor (32, E8M0)": (4.25, mx(MX_OCP_FLOOR)),
        "MXFP4 ceil (32, E8M0)": (4.25, mx(MX_CEIL)),
        "INT4 (16, E4M3 + fp32)": (4.5, i4(16, INT4_E4M3_TENSOR)),
        "INT4 (32, E8M0)": (4.25, i4(32, INT4_E8M0)),
        "INT4 (128, bf16)": (4.125, i4(128, INT4_BF16)),
        "INT4 (per row, fp32)": (4.0 + 32.0 / cols, i4(cols, INT4_F32)),
    }


def sqnr_db(x: np.ndarray, y: np.ndarray) -> float:
    x = np.asarray(x, np.float64)
    err = np.sum((x - y) ** 2)
    return float("inf") if err == 0 else float(10.0 * np.log10(np.sum(x * x) / err))


def run(rows: int = 512, cols: int = 4096, seed: int = 0, gemm_rows: int = 32):
    """Rows of results: dict(dist, format, bits, sqnr_db, small_sqnr_db, gemm_rel_err)."""
    from synthetic import activations_f32, heavy_tailed, to_bf16_bits

    a = bf16_bits_to_f64(to_bf16_bits(activations_f32(gemm_rows, cols, 0.005, 30.0, seed + 100)))
    out = []
    for di, dist in enumerate(DISTRIBUTIONS):
        x = heavy_tailed(rows, cols, dist, seed + di)
        xd = x.astype(np.float64)
        small = np.abs(xd) <= np.median(np.abs(xd))
        c_ref = a @ xd.T
        for name, (bits, q) in _formats(cols).items():
            y = q(x)
            c = a @ y.T
            out.append(dict(dist=dist, format=name, bits=bits, sqnr_db=sqnr_db(xd, y),
                            small_sqnr_db=sqnr_db(xd[small], y[small]),
                            gemm_rel_err=float(np.linalg.norm(c - c_ref) / np.linalg.norm(c_ref))))
    return out


def table(results) -> str:
    lines = ["| distribution | format (block, step) | bits/value | SQNR dB | SQNR dB, \\|x\\| <= median | W4A16 rel. error |",
             "|---|---|---|---|---|---|"]
    for r in results:
        lines.append(f"| {r['dist']} | {r['format']} | {r['bits']:.3f} | {r['sqnr_db']:.2f} | "
                     f"{r['small_sqnr_db']:.2f} | {r['gemm_rel_err']:.4f} |")
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--rows", type=int, default=512)
    ap.add_argument("--cols", type=int, default=4096)
    ap.add_argument("--seed", type=int, default=0)
    args = ap.parse_args()
    print(table(run(args.rows, args.cols, args.seed)))


if __name__ == "__main__":
    main()
