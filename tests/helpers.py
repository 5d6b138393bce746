"""Shared helpers for the GPU parity tests (test infrastructure)."""
from __future__ import annotations

import sys

import numpy as np
import torch

GEMM_RTOL = 2e-3   # |C - C_ref| <= 2e-3 * sum_k |a w|, per element, for the fp32 result
BF16_HALF_ULP_REL = 2.0 ** -8   # rounding an fp32 value to bf16 moves it by at most 2^-8 of itself


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev() -> torch.device:
    return torch.device("cuda:0")


def f32_to_dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev())


def bf16bits_to_dev(b: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(b, np.uint16).view(np.int16)).view(torch.bfloat16).to(dev())


def bf16_tensor_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def assert_bytes_equal(got: torch.Tensor, want: np.ndarray, what: str) -> None:
    g = got.detach().cpu().numpy()
    assert g.shape == want.shape, (what, g.shape, want.shape)
    bad = np.argwhere(g != want)
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {bad[:3].tolist()}: got {g[tuple(bad[0])]} want {want[tuple(bad[0])]}"


def gemm_out_f64(c: torch.Tensor) -> np.ndarray:
    return c.detach().float().cpu().numpy().astype(np.float64)


def assert_gemm_close(c: torch.Tensor | np.ndarray, ref: np.ndarray, tol: np.ndarray, what: str) -> None:
    """fp32 outputs: |C - C_ref| <= 2e-3 * sum|a w|.  bf16 outputs are that fp32
    result rounded to nearest even, so bf16's own half ulp (<= 2^-8 |C|) is added."""
    is_bf16 = isinstance(c, torch.Tensor) and c.dtype == torch.bfloat16
    got = gemm_out_f64(c) if isinstance(c, torch.Tensor) else c
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    err = np.abs(got - ref)
    lim = GEMM_RTOL * tol
    if is_bf16:
        lim = lim * (1 + BF16_HALF_ULP_REL) + BF16_HALF_ULP_REL * np.abs(ref)
    bad = err > lim
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside 2e-3*sum|aw|; worst ratio "
                           f"{(err / np.maximum(lim, 1e-300)).max():.3g}")
    assert np.isfinite(got).all(), what


def sample_rows(M: int, n: int = 256, seed: int = 0) -> np.ndarray:
    """Rows 0 and M - 1 and n distinct others, drawn with a seeded generator, sorted."""
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, M - 1], rng.choice(M, min(n, M), replace=False)]))


def assert_bf16_is_rounded(c_bf16: torch.Tensor, c_f32: torch.Tensor, what: str) -> None:
    """A bf16 output equals the fp32 output of the same call rounded to nearest even,
    element for element (the kernels accumulate in fp32 the same way for both)."""
    assert c_bf16.dtype == torch.bfloat16 and c_f32.dtype == torch.float32
    want = c_f32.to(torch.bfloat16)
    same = c_bf16.view(torch.int16) == want.view(torch.int16)
    if not bool(same.all()):
        bad = (~same).nonzero()[:3].tolist()
        raise AssertionError(f"{what}: {int((~same).sum())} bf16 outputs differ from the rounded fp32 "
                             f"output, first at {bad}")
