"""The allocation-free W4A4 entry point, gemm_w4a4_noalloc, against gemm_w4a4.

gemm_w4a4_noalloc is gemm_w4a4 with A's packed NVFP4 form kept in the library's
own device scratch instead of a caller's workspace; the two share every kernel,
so their outputs must be equal bit for bit (beyond the 2e-3 * sum|a w| GEMM bar
both meet against the oracle).  Checked on two calls in a row, the second with
a smaller input, in both activation-scale modes, plus the scratch-size refusal
and that the calls allocate no device memory through torch's allocator.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import assert_gemm_close, bf16bits_to_dev, dev, log
from synthetic import activations_f32, to_bf16_bits, weights

pytestmark = pytest.mark.gpu

FP4_ERR_WORKSPACE = 5


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def fp4():
    import block_scaled_fp4_04_amd as m

    return m


def _weight(N, K, seed):
    w = weights(N, K, 0.02, 0.001, 20.0, seed=seed)
    oc, os_, ot = oracle.nvfp4_quantize(w)
    p = fp4().PackedNVFP4(torch.from_numpy(oc).to(dev()), torch.from_numpy(os_).to(dev()),
                          torch.from_numpy(ot).to(dev()), N, K, False)
    return p, (oc, os_, ot)


@pytest.mark.parametrize("mode", ["row", "tensor"])
def test_noalloc_equals_workspace_entry_point_twice(mode):
    m = fp4()
    N, K = 700, 2048
    wp, (oc, os_, ot) = _weight(N, K, seed=5)
    for call, M in enumerate((1000, 37)):            # the second call is smaller
        log(f"gemm_w4a4_noalloc call {call} M={M} N={N} K={K} mode={mode}")
        a_bits = to_bf16_bits(activations_f32(M, K, 0.005, 30.0, seed=100 + call))
        a = bf16bits_to_dev(a_bits)
        out = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev())
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        m.gemm_w4a4_noalloc(a, wp, a_mode=mode, out=out)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        ref = m.gemm_w4a4(a, wp, a_mode=mode, dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"call {call}: differs from gemm_w4a4"
        c_ref, tol = oracle.gemm_w4a4_ref(a_bits, oc, os_, ot, a_per_row=(mode == "row"))
        assert_gemm_close(out, c_ref, tol, f"noalloc call {call} vs oracle")


def test_noalloc_full_workload_shape_bf16():
    """M = 4096, K = 5120 (11.8 MB of scratch), bf16 output, against gemm_w4a4."""
    m = fp4()
    N, K, M = 1024, 5120, 4096
    wp, _ = _weight(N, K, seed=8)
    a = bf16bits_to_dev(to_bf16_bits(activations_f32(M, K, 0.005, 30.0, seed=9)))
    c1 = m.gemm_w4a4_noalloc(a, wp)
    c2 = m.gemm_w4a4(a, wp)
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))


def test_noalloc_refuses_inputs_past_its_scratch():
    m = fp4()
    L = m.lib()
    K = 5120
    M = 12000                                        # A's packed form needs 34.6 MB > 32 MiB
    assert L.gemm_w4a4_workspace(M, K, 1) > 32 << 20
    wp, _ = _weight(64, K, seed=3)
    a = torch.zeros(M, K, dtype=torch.bfloat16, device=dev())
    with pytest.raises(m.Fp4Error) as e:
        m.gemm_w4a4_noalloc(a, wp)
    assert e.value.status == FP4_ERR_WORKSPACE
    M2 = 6000                                        # 17.3 MB: accepted
    assert L.gemm_w4a4_workspace(M2, K, 1) <= 32 << 20
    c = m.gemm_w4a4_noalloc(a[:M2], wp, dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.all(c == 0)
