"""Pins of the oracle's grouped (mixture-of-experts) GEMM references.

A grouped row t of group e is A[row_index[t]] . W_e^T (edge-FP4 article,
eefocus.com, "FP4 as the next core standard": MoE expert weights in MXFP4;
Unsloth Dynamic NVFP4 article, aixq.cc, throughput section: a mixture-of-experts
model with NVFP4 weights).  The references are pinned against a brute-force sum
in token space (every (token, slot) pair computed from decoded bytes by plain
loops, without the grouped layout), against the dense references with a single
group, and the grouping itself against its definition.
"""
import numpy as np
import pytest

import oracle
from synthetic import MOE_WORKLOADS, activations_f32, group_by_expert, moe_routing, to_bf16_bits, weights


def _decode_nv(codes, scales, tscale):
    """Brute-force NVFP4 decode of one [N, K] weight: E2M1 x E4M3 x tensor scale."""
    N, K = codes.shape[0], codes.shape[1] * 2
    w = np.empty((N, K))
    for n in range(N):
        for k in range(K):
            c = (codes[n, k // 2] >> (4 * (k % 2))) & 15
            w[n, k] = oracle.e2m1_decode(int(c)) * oracle.e4m3_decode(int(scales[n, k // 16])) * float(tscale)
    return w


def _decode_mx(codes, scales):
    N, K = codes.shape[0], codes.shape[1] * 2
    w = np.empty((N, K))
    for n in range(N):
        for k in range(K):
            c = (codes[n, k // 2] >> (4 * (k % 2))) & 15
            w[n, k] = oracle.e2m1_decode(int(c)) * oracle.e8m0_decode(int(scales[n, k // 32]))
    return w


def _tiny(fmt, seed=0, T=7, E=5, top_k=2, K=64, N=3, dead=1):
    top = moe_routing(T, E, top_k, skew=0.5, dead=dead, seed=seed)
    offs, ridx, slot = group_by_expert(top, E)
    a = to_bf16_bits(activations_f32(T, K, 0.1, 8.0, seed=seed + 1))
    w = np.stack([weights(N, K, 1.0, 0.05, 10.0, seed=seed + 10 + e) for e in range(E)])
    if fmt == "mx":
        q = [oracle.mxfp4_quantize(w[e]) for e in range(E)]
        codes = np.stack([x[0] for x in q])
        scales = np.stack([x[1] for x in q])
        return top, offs, ridx, slot, a, codes, scales, None
    q = [oracle.nvfp4_quantize(w[e]) for e in range(E)]
    codes = np.stack([x[0] for x in q])
    scales = np.stack([x[1] for x in q])
    ts = np.array([x[2][0] for x in q], np.float32)
    return top, offs, ridx, slot, a, codes, scales, ts


def test_grouping_matches_its_definition():
    top = moe_routing(50, 9, 3, skew=0.7, dead=2, seed=3)
    offs, ridx, slot = group_by_expert(top, 9)
    assert offs[0] == 0 and offs[-1] == 150 and np.all(np.diff(offs) >= 0)
    assert np.all(offs[-3:] == 150)                           # the 2 dead experts own no rows
    for i in range(50):
        assert len(set(top[i])) == 3                          # distinct experts per token
        for j in range(3):
            t = slot[i, j]
            e = top[i, j]
            assert offs[e] <= t < offs[e + 1] and ridx[t] == i
    assert sorted(slot.reshape(-1).tolist()) == list(range(150))
    for e in range(9):                                        # token order within a group
        assert np.all(np.diff(ridx[offs[e]:offs[e + 1]]) > 0)


@pytest.mark.parametrize("fmt", ["nv", "mx", "nv44"])
@pytest.mark.parametrize("seed", [0, 1])
def test_grouped_ref_against_token_space_brute_force(fmt, seed):
    top, offs, ridx, slot, a, codes, scales, ts = _tiny("mx" if fmt == "mx" else "nv", seed)
    E, T, K = codes.shape[0], a.shape[0], a.shape[1]
    if fmt == "nv44":
        ac, asc, ats = oracle.nvfp4_quantize(a, per_row=True)
        av = np.empty((T, K))
        for i in range(T):
            for k in range(K):
                c = (ac[i, k // 2] >> (4 * (k % 2))) & 15
                av[i, k] = oracle.e2m1_decode(int(c)) * oracle.e4m3_decode(int(asc[i, k // 16])) * float(ats[i])
        c_ref, t_ref = oracle.nvfp4_grouped_gemm_w4a4_ref(a, codes, scales, ts, offs, ridx)
    else:
        av = oracle.bf16_bits_to_f64(a)
        if fmt == "mx":
            c_ref, t_ref = oracle.mxfp4_grouped_gemm_w4a16_ref(a, codes, scales, offs, ridx)
        else:
            c_ref, t_ref = oracle.nvfp4_grouped_gemm_w4a16_ref(a, codes, scales, ts, offs, ridx)
    wv = [_decode_mx(codes[e], scales[e]) if fmt == "mx" else _decode_nv(codes[e], scales[e], ts[e])
          for e in range(E)]
    assert c_ref.shape == (int(offs[-1]), codes.shape[1])
    for i in range(T):
        for j in range(top.shape[1]):
            e, t = top[i, j], slot[i, j]
            for n in range(codes.shape[1]):
                s = sum(av[i, k] * wv[e][n, k] for k in range(K))
                sa = sum(abs(av[i, k] * wv[e][n, k]) for k in range(K))
                assert abs(c_ref[t, n] - s) <= 1e-12 * sa
                assert abs(t_ref[t, n] - sa) <= 1e-12 * sa


def test_single_group_reduces_to_the_dense_references():
    M, K, N = 9, 128, 5
    a = to_bf16_bits(activations_f32(M, K, 0.1, 8.0, seed=4))
    w = weights(N, K, 1.0, 0.05, 10.0, seed=5)
    offs = np.array([0, M], np.int32)
    nc, ns, nt = oracle.nvfp4_quantize(w)
    mc, ms = oracle.mxfp4_quantize(w)
    got, _ = oracle.nvfp4_grouped_gemm_w4a16_ref(a, nc[None], ns[None], nt, offs)
    assert np.array_equal(got, oracle.gemm_w4a16_ref(a, nc, ns, nt)[0])
    got, _ = oracle.mxfp4_grouped_gemm_w4a16_ref(a, mc[None], ms[None], offs)
    assert np.array_equal(got, oracle.mxfp4_gemm_w4a16_ref(a, mc, ms)[0])
    got, _ = oracle.nvfp4_grouped_gemm_w4a4_ref(a, nc[None], ns[None], nt, offs)
    assert np.array_equal(got, oracle.gemm_w4a4_ref(a, nc, ns, nt, a_per_row=True)[0])


def test_sampled_rows_equal_the_full_reference():
    top, offs, ridx, slot, a, codes, scales, ts = _tiny("nv", 2, T=20, E=6, top_k=3)
    full, tf = oracle.nvfp4_grouped_gemm_w4a16_ref(a, codes, scales, ts, offs, ridx)
    rows = np.array([0, 5, 17, 33, 59])
    part, tp = oracle.nvfp4_grouped_gemm_w4a16_ref(a, codes, scales, ts, offs, ridx, rows=rows)
    assert np.array_equal(part, full[rows]) and np.array_equal(tp, tf[rows])


def test_moe_workload_shape():
    wl = MOE_WORKLOADS["moe_e128_top8_t4096_k2048_n1536"]
    top, offs, ridx, slot = wl.routing()
    loads = np.diff(offs)
    assert offs[-1] == wl.tokens * wl.top_k and loads[-4:].sum() == 0 and loads.max() < 1000
