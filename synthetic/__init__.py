"""Seeded synthetic inputs shared by the oracle-side tests, the GPU tests and the benchmark.

This module only draws random numbers and lays them out. It holds none of the
quantization or GEMM arithmetic: every input the tests and the benchmark feed to
either side comes from here, so both sides see the same bits.

Recipes (workload shapes from the NVFP4 wiki page, section "Technical principle",
and from the decode / prefill split in the edge-FP4 article, section on compute,
memory and precision; the pages print no layer shapes, so K = 5120, N = 17408 are
the workload's stated sizes):

* weights: ``standard_normal(float32) * sigma``; a Bernoulli(p) mask per entry,
  masked entries multiplied by ``factor`` (bell-shaped with outliers).
* activations: ``standard_normal(float32)``; optionally a Bernoulli(p) mask per
  K-column, masked columns multiplied by ``factor``; then cast to bfloat16 with
  round-to-nearest-even (torch's CPU cast).

All generators use numpy's PCG64 ``default_rng(seed)``.
"""
from __future__ import annotations

import dataclasses

import numpy as np

__all__ = [
    "weights",
    "activations_f32",
    "to_bf16_bits",
    "bf16_bits_to_f32",
    "Workload",
    "WORKLOADS",
]


def weights(rows: int, cols: int, sigma: float = 1.0, outlier_p: float = 0.0,
            outlier_factor: float = 1.0, seed: int = 0) -> np.ndarray:
    """fp32 [rows, cols] ~ N(0, sigma^2) with per-entry Bernoulli(p) outliers x factor."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((rows, cols), dtype=np.float32)
    if sigma != 1.0:
        w *= np.float32(sigma)
    if outlier_p > 0.0:
        mask = rng.random((rows, cols)) < outlier_p
        w[mask] *= np.float32(outlier_factor)
    return w


def activations_f32(rows: int, cols: int, channel_p: float = 0.0,
                    channel_factor: float = 1.0, seed: int = 1) -> np.ndarray:
    """fp32 [rows, cols] ~ N(0, 1); Bernoulli(p) K-channels (columns) scaled by factor."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((rows, cols), dtype=np.float32)
    if channel_p > 0.0:
        cmask = rng.random(cols) < channel_p
        a[:, cmask] *= np.float32(channel_factor)
    return a


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns (uint16), rounded to nearest even by torch's CPU cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> fp32 (exact widening)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: tuple
    K: int
    N: int
    w_sigma: float
    w_outlier_p: float
    w_outlier_factor: float
    a_channel_p: float = 0.0
    a_channel_factor: float = 1.0
    w_seed: int = 0
    a_seed: int = 1

    def weights(self, rows: int | None = None) -> np.ndarray:
        """The workload's fp32 weights; ``rows`` < N draws the same generator and keeps the first rows."""
        w = weights(self.N, self.K, self.w_sigma, self.w_outlier_p, self.w_outlier_factor,
                    self.w_seed)
        return w if rows is None else w[:rows].copy()

    def activations_bf16(self, m: int) -> np.ndarray:
        return to_bf16_bits(activations_f32(m, self.K, self.a_channel_p,
                                            self.a_channel_factor, self.a_seed))


# The five workloads.  Names say what each is, with its sizes.
WORKLOADS = {
    # tiny NVFP4 round trip + W4A16: W 256x256 ~N(0,1), 1% entries x10; A 4x256; seed 0
    "tiny_roundtrip_256": Workload("tiny_roundtrip_256", (4,), 256, 256, 1.0, 0.01, 10.0,
                                   w_seed=0, a_seed=0),
    # W4A16 decode GEMV: K=5120, N=17408, W ~N(0, 0.02^2), 0.1% x20; M in {1, 4, 16}
    "decode_gemv_k5120_n17408": Workload("decode_gemv_k5120_n17408", (1, 4, 16), 5120, 17408,
                                         0.02, 0.001, 20.0),
    # W4A16 prefill GEMM: M=4096; A has 0.5% K-channels x30
    "prefill_w4a16_m4096": Workload("prefill_w4a16_m4096", (4096,), 5120, 17408, 0.02, 0.001,
                                    20.0, 0.005, 30.0),
    # W4A4 prefill: same inputs, A quantized per row on the GPU
    "prefill_w4a4_m4096": Workload("prefill_w4a4_m4096", (4096,), 5120, 17408, 0.02, 0.001,
                                   20.0, 0.005, 30.0),
    # MXFP4 vs NVFP4 W4A4 at M=8192 on identical bf16 inputs
    "mx_vs_nv_w4a4_m8192": Workload("mx_vs_nv_w4a4_m8192", (8192,), 5120, 17408, 0.02, 0.001,
                                    20.0, 0.005, 30.0),
}
