"""GPU parity of the grouped (mixture-of-experts) GEMMs.

Grouped row t of group e is C[t] = A[row_index[t]] . W_e^T (edge-FP4 article,
eefocus.com, "FP4 as the next core standard": MoE expert weights in MXFP4;
Unsloth Dynamic NVFP4 article, aixq.cc, throughput section: a mixture-of-experts
model with NVFP4 weights, W4A16 and all-W4A4).  Every output element must meet
|C - C_ref| <= 2e-3 * sum_k |a w| against the oracle's fp64 grouped reference
(NVFP4 W4A16, MXFP4 W4A16, NVFP4 W4A4 with per-row activation quantization),
with the router's permutation applied inside the kernel (row_index) or the
activations already in grouped order; uneven and empty groups, groups larger than
a tile, K with a ragged number of pipeline stages, N not a multiple of the tile,
both tile heights, and sampled rows at the full workload size.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import assert_bf16_is_rounded, assert_gemm_close, bf16bits_to_dev, dev, log
from synthetic import MOE_WORKLOADS, activations_f32, group_by_expert, moe_routing, to_bf16_bits, weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def fp4():
    import block_scaled_fp4_04_amd as m

    return m


def _i32(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.int32)).to(dev())


def _experts(fmt, E, N, K, seed):
    w = np.stack([weights(N, K, 0.02, 0.001, 20.0, seed=seed + e) for e in range(E)])
    if fmt == "mx":
        q = [oracle.mxfp4_quantize(w[e]) for e in range(E)]
        codes, scales = np.stack([x[0] for x in q]), np.stack([x[1] for x in q])
        dw = fp4().ExpertsMXFP4(torch.from_numpy(codes).to(dev()), torch.from_numpy(scales).to(dev()), E, N, K)
        return codes, scales, None, dw
    q = [oracle.nvfp4_quantize(w[e]) for e in range(E)]
    codes, scales = np.stack([x[0] for x in q]), np.stack([x[1] for x in q])
    ts = np.array([x[2][0] for x in q], np.float32)
    dw = fp4().ExpertsNVFP4(torch.from_numpy(codes).to(dev()), torch.from_numpy(scales).to(dev()),
                            torch.from_numpy(ts).to(dev()), E, N, K)
    return codes, scales, ts, dw


def _run(fmt, a, dw, offs, ridx, dtype):
    m = fp4()
    go = _i32(offs)
    ri = None if ridx is None else _i32(ridx)
    ad = bf16bits_to_dev(a)
    if fmt == "nv16":
        return m.nvfp4_grouped_gemm_w4a16(ad, dw, go, ri, dtype=dtype)
    if fmt == "mx":
        return m.mxfp4_grouped_gemm_w4a16(ad, dw, go, ri, dtype=dtype)
    return m.nvfp4_grouped_gemm_w4a4(ad, dw, go, ri, dtype=dtype)


def _ref(fmt, a, codes, scales, ts, offs, ridx, rows=None):
    if fmt == "nv16":
        return oracle.nvfp4_grouped_gemm_w4a16_ref(a, codes, scales, ts, offs, ridx, rows)
    if fmt == "mx":
        return oracle.mxfp4_grouped_gemm_w4a16_ref(a, codes, scales, offs, ridx, rows)
    return oracle.nvfp4_grouped_gemm_w4a4_ref(a, codes, scales, ts, offs, ridx, rows)


# (tokens, experts, top_k, K, N, router skew, empty experts)
CASES = [
    (7, 5, 2, 128, 40, 0.5, 1),        # a handful of rows per group, N inside one tile
    (300, 8, 2, 256, 300, 0.3, 1),     # ~75 rows per group, N over two tiles
    (600, 6, 3, 384, 520, 0.3, 0),     # groups over 128 rows (2-4 row tiles), 6 / 3 ring stages
    (1200, 4, 2, 640, 260, 0.2, 0),    # ~600 rows per group: 256-row tiles
    (50, 16, 4, 1152, 64, 1.0, 3),     # many small and empty groups, 18 / 9 stages
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("fmt", ["nv16", "mx", "nv44"])
@pytest.mark.parametrize("gather", [True, False])
def test_grouped_gemm(case, fmt, gather):
    T, E, k, K, N, skew, dead = case
    log(f"grouped {fmt} T={T} E={E} top{k} K={K} N={N} gather={gather}")
    top = moe_routing(T, E, k, skew, dead, seed=T + E)
    offs, ridx, _ = group_by_expert(top, E)
    a = to_bf16_bits(activations_f32(T, K, 0.005, 30.0, seed=K))
    if not gather:                                     # A already in grouped order
        a, ridx = a[ridx], None
    codes, scales, ts, dw = _experts("mx" if fmt == "mx" else "nv", E, N, K, seed=7 * E + N)
    c = _run(fmt, a, dw, offs, ridx, torch.float32)
    torch.cuda.synchronize()
    ref, tol = _ref(fmt, a, codes, scales, ts, offs, ridx)
    assert_gemm_close(c, ref, tol, f"grouped {fmt} {case}")


@pytest.mark.parametrize("fmt", ["nv16", "mx", "nv44"])
def test_grouped_bf16_output_and_one_busy_group(fmt):
    """All rows in one group (between empty ones); bf16 C."""
    T, E, K, N = 700, 5, 256, 200
    offs = np.array([0, 0, 0, T, T, T], np.int32)
    ridx = np.random.default_rng(1).permutation(T).astype(np.int32)
    a = to_bf16_bits(activations_f32(T, K, 0.005, 30.0, seed=3))
    codes, scales, ts, dw = _experts("mx" if fmt == "mx" else "nv", E, N, K, seed=11)
    c = _run(fmt, a, dw, offs, ridx, torch.bfloat16)
    torch.cuda.synchronize()
    ref, tol = _ref(fmt, a, codes, scales, ts, offs, ridx)
    assert_gemm_close(c, ref, tol, f"grouped one busy group {fmt}")


@pytest.mark.parametrize("fmt", ["nv16", "mx", "nv44"])
def test_grouped_every_live_row_block_count(fmt):
    """Groups whose last 128-row tile holds 1, 31, 32, 33, 64, 65, 96, 97, 127, 128
    and 129 + 63 rows: each count of live 32-row blocks (1-4 of a wave's 4 in the
    W4A16 layout; 0-2 of each wave's 2 in W4A4's 2 x 2 split) and both sides of
    every block boundary, with the rows gathered and fp32 C."""
    sizes = [1, 31, 32, 33, 64, 65, 96, 97, 127, 128, 192]
    E, K, N = len(sizes), 256, 300
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    T = int(offs[-1])
    ridx = np.random.default_rng(4).permutation(T).astype(np.int32)
    a = to_bf16_bits(activations_f32(T, K, 0.005, 30.0, seed=6))
    codes, scales, ts, dw = _experts("mx" if fmt == "mx" else "nv", E, N, K, seed=13)
    c = _run(fmt, a, dw, offs, ridx, torch.float32)
    torch.cuda.synchronize()
    ref, tol = _ref(fmt, a, codes, scales, ts, offs, ridx)
    assert_gemm_close(c, ref, tol, f"grouped live row blocks {fmt}")


def test_grouped_exact_tile_multiples():
    """Groups of exactly 128 and 256 rows, N = 512: no ragged tile anywhere."""
    E, K, N = 3, 256, 512
    offs = np.array([0, 128, 384, 640], np.int32)
    a = to_bf16_bits(activations_f32(640, K, 0.005, 30.0, seed=5))
    codes, scales, ts, dw = _experts("nv", E, N, K, seed=2)
    c = _run("nv16", a, dw, offs, None, torch.float32)
    torch.cuda.synchronize()
    ref, tol = _ref("nv16", a, codes, scales, ts, offs, None)
    assert_gemm_close(c, ref, tol, "grouped exact multiples")


def test_grouped_empty_call_and_out_of_range_row_index():
    """rows == 0 is a no-op; a row index outside A reads as a zero row (C row 0)."""
    m = fp4()
    E, N, K = 2, 64, 128
    codes, scales, ts, dw = _experts("nv", E, N, K, seed=9)
    a = to_bf16_bits(activations_f32(4, K, seed=1))
    ad = bf16bits_to_dev(a)
    out = m.nvfp4_grouped_gemm_w4a16(ad, dw, _i32([0, 0, 0]), _i32(np.zeros(0, np.int32)), dtype=torch.float32)
    assert out.shape == (0, N)
    ridx = np.array([2, 9, -1, 0], np.int32)          # rows 1 and 2 point outside A
    offs = np.array([0, 2, 4], np.int32)
    c = m.nvfp4_grouped_gemm_w4a16(ad, dw, _i32(offs), _i32(ridx), dtype=torch.float32)
    torch.cuda.synchronize()
    got = c.cpu().numpy()
    assert np.all(got[1] == 0) and np.all(got[2] == 0)
    ref, tol = oracle.nvfp4_grouped_gemm_w4a16_ref(a, codes, scales, ts, offs, np.array([2, 0, 0, 0]), rows=[0, 3])
    assert_gemm_close(got[[0, 3]].astype(np.float64), ref, tol, "valid rows next to invalid ones")


@pytest.mark.parametrize("fmt", ["nv16", "mx", "nv44"])
def test_grouped_full_size_sampled(fmt):
    wl = MOE_WORKLOADS["moe_e128_top8_t4096_k2048_n1536"]
    log(f"grouped {fmt} full size {wl.name} (sampled rows vs oracle)")
    top, offs, ridx, _ = wl.routing()
    a = wl.activations_bf16()
    w = wl.expert_weights()
    m = fp4()
    wt = torch.from_numpy(w).to(dev())
    if fmt == "mx":
        dw = m.mxfp4_quantize_experts(wt)
        codes, scales, ts = dw.codes.cpu().numpy(), dw.scales.cpu().numpy(), None
    else:
        dw = m.nvfp4_quantize_experts(wt)
        codes, scales, ts = dw.codes.cpu().numpy(), dw.scales.cpu().numpy(), dw.tscale.cpu().numpy()
    del wt
    # the device-quantized weights must equal the oracle's, expert by expert (a sample)
    for e in (0, 63, 127):
        if fmt == "mx":
            wc, wsc = oracle.mxfp4_quantize(w[e])
        else:
            wc, wsc, wts = oracle.nvfp4_quantize(w[e])
            assert ts[e] == wts[0]
        assert np.array_equal(codes[e], wc) and np.array_equal(scales[e], wsc)
    c = _run(fmt, a, dw, offs, ridx, torch.float32)
    cb = _run(fmt, a, dw, offs, ridx, torch.bfloat16)
    torch.cuda.synchronize()
    assert_bf16_is_rounded(cb, c, f"grouped {fmt}")
    rng = np.random.default_rng(6)
    live = np.nonzero(np.diff(offs))[0]
    edge = np.concatenate([offs[live], offs[live + 1] - 1])          # first and last row of every group
    rows = np.unique(np.concatenate([edge, rng.choice(int(offs[-1]), 256, replace=False)]))
    ref, tol = _ref(fmt, a, codes, scales, ts, offs, ridx, rows)
    assert_gemm_close(c[torch.from_numpy(rows).to(dev())], ref, tol, f"grouped {fmt} sampled")
