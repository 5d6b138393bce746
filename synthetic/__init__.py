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
    "heavy_tailed",
    "moe_routing",
    "group_by_expert",
    "Workload",
    "MoeWorkload",
    "WORKLOADS",
    "MOE_WORKLOADS",
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


def heavy_tailed(rows: int, cols: int, kind: str, seed: int = 0) -> np.ndarray:
    """fp32 [rows, cols] from a named distribution: "gaussian" N(0, 1),
    "gaussian_outliers" N(0, 1) with 0.1% of entries x20, "student_t3" Student's t
    with 3 degrees of freedom, "laplace" Laplace(0, 1), "channel_outliers" N(0, 1)
    with 0.5% of the columns x30 (the activation recipe)."""
    rng = np.random.default_rng(seed)
    if kind == "gaussian":
        return rng.standard_normal((rows, cols), dtype=np.float32)
    if kind == "gaussian_outliers":
        return weights(rows, cols, 1.0, 0.001, 20.0, seed)
    if kind == "student_t3":
        return rng.standard_t(3.0, (rows, cols)).astype(np.float32)
    if kind == "laplace":
        return rng.laplace(0.0, 1.0, (rows, cols)).astype(np.float32)
    if kind == "channel_outliers":
        return activations_f32(rows, cols, 0.005, 30.0, seed)
    raise ValueError(kind)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns (uint16), rounded to nearest even by torch's CPU cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> fp32 (exact widening)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def moe_routing(tokens: int, experts: int, top_k: int, skew: float = 1.0, dead: int = 0,
                seed: int = 2) -> np.ndarray:
    """Top-k expert ids [tokens, top_k] (int32, distinct per token, best first).

    Router logits are N(0, 1) per (token, expert) plus a per-expert bias
    ``skew * N(0, 1)``, so expert loads are uneven; the last ``dead`` experts get
    no tokens at all."""
    rng = np.random.default_rng(seed)
    bias = rng.standard_normal(experts).astype(np.float32) * np.float32(skew)
    logits = rng.standard_normal((tokens, experts), dtype=np.float32) + bias
    if dead:
        logits[:, experts - dead:] = -np.inf
    top = np.argsort(-logits, axis=1, kind="stable")[:, :top_k]
    return top.astype(np.int32)


def group_by_expert(topk: np.ndarray, experts: int):
    """The grouped row layout of a routing: (group_offs int32 [experts + 1],
    row_index int32 [tokens * top_k] = the token of each grouped row, slot_row
    int32 [tokens, top_k] = the grouped row of each (token, slot)).  Rows of one
    expert keep token order (a stable sort of the flattened (token, slot) list)."""
    T, k = topk.shape
    flat = topk.reshape(-1).astype(np.int64)
    order = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=experts)
    offs = np.zeros(experts + 1, np.int64)
    np.cumsum(counts, out=offs[1:])
    row_index = (order // k).astype(np.int32)
    slot_row = np.empty(T * k, np.int64)
    slot_row[order] = np.arange(T * k)
    return offs.astype(np.int32), row_index, slot_row.reshape(T, k).astype(np.int32)


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


@dataclasses.dataclass(frozen=True)
class MoeWorkload:
    """A mixture-of-experts layer: `tokens` bf16 rows of width K, each routed to
    `top_k` of `experts` weights [N, K] (drawn like the dense weights, one
    generator for all experts, expert e = rows e N .. e N + N - 1)."""
    name: str
    tokens: int
    experts: int
    top_k: int
    K: int
    N: int
    w_sigma: float
    w_outlier_p: float
    w_outlier_factor: float
    a_channel_p: float = 0.0
    a_channel_factor: float = 1.0
    skew: float = 1.0
    dead: int = 0
    w_seed: int = 0
    a_seed: int = 1
    r_seed: int = 2

    def expert_weights(self) -> np.ndarray:
        w = weights(self.experts * self.N, self.K, self.w_sigma, self.w_outlier_p, self.w_outlier_factor,
                    self.w_seed)
        return w.reshape(self.experts, self.N, self.K)

    def activations_bf16(self) -> np.ndarray:
        return to_bf16_bits(activations_f32(self.tokens, self.K, self.a_channel_p, self.a_channel_factor,
                                            self.a_seed))

    def routing(self):
        """(topk, group_offs, row_index, slot_row) of the workload's router."""
        top = moe_routing(self.tokens, self.experts, self.top_k, self.skew, self.dead, self.r_seed)
        return (top,) + group_by_expert(top, self.experts)


# Mixture-of-experts workloads (the pages name MoE models and MXFP4 expert weights
# but print no layer sizes; these sizes are chosen here: 128 experts, 8 per token,
# hidden 2048, expert output 1536 (gate and up projections side by side)).
MOE_WORKLOADS = {
    # prefill-sized batch: 4096 tokens -> 32768 grouped rows, mean 256 per expert;
    # router bias skew 0.3 gives loads from 0 to 794 rows (median 229), and the
    # last 4 experts get none
    "moe_e128_top8_t4096_k2048_n1536": MoeWorkload("moe_e128_top8_t4096_k2048_n1536", 4096, 128, 8, 2048, 1536,
                                                   0.02, 0.001, 20.0, 0.005, 30.0, skew=0.3, dead=4),
}
