"""Host-side checks of the C ABI (CPU only; no kernel is ever launched here).

The library must build for gfx950, load, export every function include/fp4blk.h
declares, and reject bad arguments with its documented status codes before it
touches a device.  With valid arguments and no GPU it reports FP4_ERR_NO_DEVICE.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4blk.h")

OK, NULL, SHAPE, LAYOUT, DTYPE, WORKSPACE, NO_DEVICE, UNSUPPORTED, HIP = range(9)

FAKE = 1 << 20  # a 16-byte-aligned non-null address; never dereferenced on the host


def _declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    names = re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", txt)
    skip = {"if", "defined", "sizeof"}
    return sorted(set(n for n in names if n not in skip))


@pytest.fixture(scope="module")
def L():
    import block_scaled_fp4_04_amd as fp4

    if not os.path.exists(fp4.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    return fp4.lib()


def test_exports_every_declared_symbol(L):
    import block_scaled_fp4_04_amd as fp4

    declared = _declared_functions()
    assert len(declared) >= 16
    for name in declared:
        assert hasattr(L, name), f"libfp4blk.so does not export {name}"
    assert set(declared) == set(fp4.exported_names())


def test_single_hip_runtime_in_process(L):
    maps = open("/proc/self/maps").read()
    libs = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(libs) == 1, libs


def test_status_strings(L):
    import block_scaled_fp4_04_amd as fp4

    for s in range(9):
        assert fp4.status_str(s).startswith("FP4_")
    assert "unknown" in fp4.status_str(99)


def test_version_and_no_device(L):
    assert L.fp4blk_version() == 10000
    import torch

    if not torch.cuda.is_available():
        assert L.fp4blk_check_device() == NO_DEVICE


def test_workspace_queries(L):
    assert L.nvfp4_quantize_workspace(10, 32, 0) == 4096
    assert L.nvfp4_quantize_workspace(10, 32, 1) == 0
    M, K = 4096, 5120
    co, so, to = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    L.gemm_w4a4_workspace_offsets(M, K, ctypes.byref(co), ctypes.byref(so), ctypes.byref(to))
    assert co.value == 0 and so.value == M * K // 2 and to.value == M * K // 2 + M * K // 16
    assert L.gemm_w4a4_workspace(M, K, 1) == to.value + 4 * M
    assert L.mxfp4_gemm_w4a4_workspace(M, K) == M * K // 2 + M * K // 32


def _q(L, **kw):
    a = dict(x=FAKE, xt=0, rows=4, cols=32, ldx=32, codes=FAKE, scales=FAKE, tscale=FAKE, mode=0,
             ws=FAKE, ws_bytes=4096, nonfinite=None, stream=None)
    a.update(kw)
    return L.nvfp4_quantize(*a.values())


def test_nvfp4_quantize_validation(L):
    import torch

    assert _q(L, x=None) == NULL
    assert _q(L, codes=None) == NULL
    assert _q(L, tscale=None) == NULL
    assert _q(L, cols=24, ldx=24) == SHAPE          # not a whole number of 16-blocks
    assert _q(L, rows=0) == SHAPE
    assert _q(L, cols=-16) == SHAPE
    assert _q(L, ldx=16) == LAYOUT                  # ld < cols
    assert _q(L, x=FAKE + 4) == LAYOUT              # misaligned base
    assert _q(L, xt=1, ldx=36) == LAYOUT            # bf16 rows not 16-byte aligned
    assert _q(L, xt=7) == DTYPE
    assert _q(L, mode=3) == DTYPE
    assert _q(L, ws=None) == WORKSPACE
    assert _q(L, ws_bytes=100) == WORKSPACE
    if not torch.cuda.is_available():
        assert _q(L) == NO_DEVICE
        assert _q(L, mode=1, ws=None, ws_bytes=0) == NO_DEVICE   # per-row mode needs no workspace


def test_gemm_validation(L):
    import torch

    args = dict(a=FAKE, M=4, K=64, lda=64, wc=FAKE, ws=FAKE, wt=FAKE, N=32, c=FAKE, ct=1, ldc=32,
                stream=None)

    def g(**kw):
        a = dict(args)
        a.update(kw)
        return L.gemm_w4a16(*a.values())

    assert g(a=None) == NULL
    assert g(wt=None) == NULL
    assert g(c=None) == NULL
    assert g(K=40, lda=40) == SHAPE
    assert g(M=0) == SHAPE
    assert g(N=-1) == SHAPE
    assert g(lda=32) == LAYOUT
    assert g(ldc=16) == LAYOUT
    assert g(ct=5) == DTYPE
    if not torch.cuda.is_available():
        assert g() == NO_DEVICE

    def g4(**kw):
        a = dict(a=FAKE, M=4, K=64, lda=64, mode=1, wc=FAKE, ws=FAKE, wt=FAKE, N=32, c=FAKE, ct=1,
                 ldc=32, work=FAKE, work_bytes=1 << 20, stream=None)
        a.update(kw)
        return L.gemm_w4a4(*a.values())

    assert g4(work=None) == WORKSPACE
    assert g4(work_bytes=16) == WORKSPACE
    assert g4(mode=2) == DTYPE
    if not torch.cuda.is_available():
        assert g4() == NO_DEVICE

    def g4s(**kw):
        a = dict(a=FAKE, M=8, K=256, lda=256, mode=1, wc=FAKE, ws=FAKE, wt=FAKE, N=32, c=FAKE, ct=0,
                 ldc=32, work=FAKE, work_bytes=1 << 20, stream=None)
        a.update(kw)
        return L.gemm_w4a4_seg(*a.values())

    assert g4s(K=64, lda=64) == SHAPE       # whole 128-element segments
    assert g4s(wt=None) == NULL
    assert g4s(work_bytes=16) == WORKSPACE

    def p4s(**kw):
        a = dict(ac=FAKE, asc=FAKE, at=FAKE, mode=1, M=8, K=256, wc=FAKE, ws=FAKE, wt=FAKE, N=32, c=FAKE,
                 ct=1, ldc=32, stream=None)
        a.update(kw)
        return L.gemm_nvfp4_w4a4_prequant_seg(*a.values())

    assert p4s(K=192) == SHAPE
    assert p4s(at=None) == NULL
    assert p4s(mode=5) == DTYPE
    # A or W codes of 2^31 bytes or more (K = 5120: 838,861 rows) are refused on
    # the host, before A is quantized
    big = dict(K=5120, lda=5120, work_bytes=1 << 40)
    assert g4s(M=838861, ldc=32, **big) == SHAPE and g4s(N=838861, ldc=838861, **big) == SHAPE
    assert p4s(M=838861, K=5120) == SHAPE and p4s(N=838861, K=5120, ldc=838861) == SHAPE
    if not torch.cuda.is_available():
        assert g4s() == NO_DEVICE and p4s() == NO_DEVICE
        assert g4s(M=838860, **big) == NO_DEVICE    # just under the limit


def test_decode_layout_validation(L):
    import torch

    def pk(**kw):
        a = dict(codes=FAKE, scales=FAKE, N=32, K=256, cp=FAKE, sp=FAKE, stream=None)
        a.update(kw)
        return L.nvfp4_pack_decode(*a.values())

    assert pk(codes=None) == NULL
    assert pk(sp=None) == NULL
    assert pk(K=192) == SHAPE          # not whole 128-element segments
    assert pk(N=0) == SHAPE
    assert pk(cp=FAKE + 8) == LAYOUT
    if not torch.cuda.is_available():
        assert pk() == NO_DEVICE

    def gd(**kw):
        a = dict(a=FAKE, M=4, K=256, lda=256, wc=FAKE, ws=FAKE, wt=FAKE, N=32, c=FAKE, ct=1, ldc=32,
                 stream=None)
        a.update(kw)
        return L.gemm_w4a16_decode(*a.values())

    assert gd(a=None) == NULL
    assert gd(wt=None) == NULL
    assert gd(K=192, lda=192) == SHAPE
    assert gd(M=17, K=192, lda=192) == SHAPE
    assert gd(lda=128) == LAYOUT
    assert gd(ws=FAKE + 4) == LAYOUT
    assert gd(ct=9) == DTYPE
    # 32-bit byte offsets in both kernels: refused for every M, before any device call
    assert gd(M=1, K=8192, lda=8192, N=524288, ldc=524288) == SHAPE          # weight codes of exactly 2 GiB
    assert gd(M=1, K=8192, lda=8192, N=1048576, ldc=1048576) == SHAPE         # 4 GiB: sizes would wrap
    assert gd(M=16, K=256, lda=1 << 26) == SHAPE                 # A spans 15 * 2^27 bytes
    assert gd(M=17, K=256, lda=1 << 26) == SHAPE
    assert L.mxfp4_gemm_w4a16_decode(FAKE, 1, 8192, 8192, FAKE, FAKE, 524288, FAKE, 1, 524288, None) == SHAPE
    assert L.mxfp4_gemm_w4a16_decode(FAKE, 4, 256, 1 << 28, FAKE, FAKE, 32, FAKE, 1, 32, None) == SHAPE
    if not torch.cuda.is_available():
        # any K % 128 == 0 at every M (the GEMV runs K past 8192 in chunks)
        assert gd() == NO_DEVICE and gd(M=17) == NO_DEVICE and gd(M=4096, K=8320, lda=8320) == NO_DEVICE
        assert gd(K=8320, lda=8320) == NO_DEVICE and gd(M=16, K=28672, lda=28672) == NO_DEVICE
        # just under the limits
        assert gd(M=1, K=8192, lda=8192, N=524287, ldc=524287) == NO_DEVICE
        assert gd(M=2, K=256, lda=(1 << 29) - 256) == NO_DEVICE


def test_mxfp4_validation(L):
    import torch

    def q(**kw):
        a = dict(x=FAKE, xt=1, rows=2, cols=64, ldx=64, codes=FAKE, scales=FAKE, rule=0,
                 nonfinite=None, stream=None)
        a.update(kw)
        return L.mxfp4_quantize(*a.values())

    assert q(cols=48, ldx=48) == SHAPE              # MXFP4 needs whole 32-blocks
    assert q(rule=2) == DTYPE
    assert q(scales=None) == NULL

    def g(**kw):
        a = dict(a=FAKE, M=8, K=96, lda=96, rule=0, wc=FAKE, ws=FAKE, N=16, c=FAKE, ct=0, ldc=16,
                 work=FAKE, work_bytes=1 << 20, stream=None)
        a.update(kw)
        return L.mxfp4_gemm_w4a4(*a.values())

    assert g(K=80, lda=80) == SHAPE
    assert g(work_bytes=10) == WORKSPACE
    if not torch.cuda.is_available():
        assert q() == NO_DEVICE and g() == NO_DEVICE


def test_mxfp4_w4a16_validation(L):
    import torch

    def g(**kw):
        a = dict(a=FAKE, M=8, K=256, lda=256, wc=FAKE, ws=FAKE, N=16, c=FAKE, ct=1, ldc=16, stream=None)
        a.update(kw)
        return L.mxfp4_gemm_w4a16(*a.values())

    assert g(a=None) == NULL
    assert g(K=96, lda=96) == SHAPE                  # K % 128 == 0
    assert g(lda=128) == LAYOUT
    assert g(ct=5) == DTYPE

    def pk(**kw):
        a = dict(codes=FAKE, scales=FAKE, N=32, K=256, cp=FAKE, sp=FAKE, stream=None)
        a.update(kw)
        return L.mxfp4_pack_decode(*a.values())

    assert pk(scales=None) == NULL
    assert pk(K=160) == SHAPE

    def gd(**kw):
        a = dict(a=FAKE, M=4, K=256, lda=256, wc=FAKE, ws=FAKE, N=32, c=FAKE, ct=1, ldc=32, stream=None)
        a.update(kw)
        return L.mxfp4_gemm_w4a16_decode(*a.values())

    assert gd(M=40, K=96, lda=96) == SHAPE
    assert gd(c=None) == NULL
    if not torch.cuda.is_available():
        assert g() == NO_DEVICE and pk() == NO_DEVICE and gd() == NO_DEVICE
        assert gd(M=17) == NO_DEVICE and gd(M=300, K=8320, lda=8320) == NO_DEVICE
        assert gd(K=8320, lda=8320) == NO_DEVICE  # the GEMV takes K past 8192 in chunks


def test_mxfp4_segment_major_gemm_validation(L):
    import torch

    assert L.mxfp4_gemm_w4a4_seg_workspace(4096, 5120) == L.mxfp4_gemm_w4a4_workspace(4096, 5120)
    assert L.mxfp4_gemm_w4a4_seg_workspace(0, 128) == 0

    def g(**kw):
        a = dict(a=FAKE, M=8, K=256, lda=256, rule=0, wc=FAKE, ws=FAKE, N=16, c=FAKE, ct=0, ldc=16,
                 work=FAKE, work_bytes=1 << 20, stream=None)
        a.update(kw)
        return L.mxfp4_gemm_w4a4_seg(*a.values())

    assert g(K=96, lda=96) == SHAPE                  # whole 128-element segments
    assert g(lda=128) == LAYOUT
    assert g(rule=3) == DTYPE
    assert g(wc=None) == NULL
    assert g(work_bytes=100) == WORKSPACE
    assert g(work=FAKE + 4) == WORKSPACE             # 16-byte aligned
    assert g(ldc=8) == LAYOUT

    def p(**kw):
        a = dict(ac=FAKE, asc=FAKE, M=8, K=256, wc=FAKE, ws=FAKE, N=16, c=FAKE, ct=1, ldc=16, stream=None)
        a.update(kw)
        return L.mxfp4_gemm_prequant_seg(*a.values())

    assert p(K=160) == SHAPE
    assert p(asc=None) == NULL
    assert p(M=0) == SHAPE
    assert p(ct=4) == DTYPE
    # codes of 2^31 bytes or more (K = 5120: 838,861 rows), refused before A is quantized
    big = dict(K=5120, lda=5120, work_bytes=1 << 40)
    assert g(M=838861, **big) == SHAPE and g(N=838861, ldc=838861, **big) == SHAPE
    assert p(M=838861, K=5120) == SHAPE and p(N=838861, K=5120, ldc=838861) == SHAPE
    if not torch.cuda.is_available():
        assert g() == NO_DEVICE and p() == NO_DEVICE
        assert g(M=838860, **big) == NO_DEVICE and p(M=838860, K=5120) == NO_DEVICE


def test_w4a8_segment_major_validation(L):
    import torch

    def g(**kw):
        a = dict(a=FAKE, M=8, K=256, lda=256, rule=0, wc=FAKE, ws=FAKE, N=16, c=FAKE, ct=0, ldc=16,
                 work=FAKE, work_bytes=1 << 20, stream=None)
        a.update(kw)
        return L.mxfp4_gemm_w4a8_seg(*a.values())

    assert g(K=192, lda=192) == SHAPE
    assert g(rule=7) == DTYPE
    assert g(work_bytes=16) == WORKSPACE
    assert g(wc=None) == NULL

    def p(**kw):
        a = dict(ac=FAKE, asc=FAKE, M=8, K=256, wc=FAKE, ws=FAKE, N=16, c=FAKE, ct=1, ldc=16, stream=None)
        a.update(kw)
        return L.mxfp4_gemm_w4a8_prequant_seg(*a.values())

    assert p(K=64) == SHAPE
    assert p(ws=None) == NULL
    assert p(ldc=15) == LAYOUT
    # MXFP8 A of 2^31 bytes or more (K = 5120: 419,431 rows) or W codes past it,
    # refused before A is quantized
    big = dict(K=5120, lda=5120, work_bytes=1 << 40)
    assert g(M=419431, **big) == SHAPE and g(N=838861, ldc=838861, **big) == SHAPE
    assert p(M=419431, K=5120) == SHAPE
    if not torch.cuda.is_available():
        assert g() == NO_DEVICE and p() == NO_DEVICE
        assert g(M=419430, **big) == NO_DEVICE and p(M=419430, K=5120) == NO_DEVICE


def test_w4a8_validation(L):
    import torch

    def q(**kw):
        a = dict(x=FAKE, xt=1, rows=2, cols=64, ldx=64, codes=FAKE, scales=FAKE, rule=0,
                 nonfinite=None, stream=None)
        a.update(kw)
        return L.mxfp8_quantize(*a.values())

    assert q(cols=48, ldx=48) == SHAPE
    assert q(rule=3) == DTYPE
    assert q(codes=None) == NULL
    assert L.mxfp4_gemm_w4a8_workspace(4, 256) == 1024 + 256
    assert L.mxfp4_gemm_w4a8_workspace(0, 256) == 0

    def g(**kw):
        a = dict(a=FAKE, M=8, K=256, lda=256, rule=0, wc=FAKE, ws=FAKE, N=16, c=FAKE, ct=0, ldc=16,
                 work=FAKE, work_bytes=1 << 20, stream=None)
        a.update(kw)
        return L.mxfp4_gemm_w4a8(*a.values())

    assert g(K=96, lda=96) == SHAPE                   # K % 128 == 0
    assert g(work_bytes=100) == WORKSPACE
    assert g(rule=7) == DTYPE

    def gp(**kw):
        a = dict(ac=FAKE, asc=FAKE, M=8, K=256, wc=FAKE, ws=FAKE, N=16, c=FAKE, ct=0, ldc=16, stream=None)
        a.update(kw)
        return L.mxfp4_gemm_w4a8_prequant(*a.values())

    assert gp(ac=None) == NULL
    assert gp(K=160) == SHAPE
    if not torch.cuda.is_available():
        assert q() == NO_DEVICE and g() == NO_DEVICE and gp() == NO_DEVICE


def test_grouped_validation(L):
    import torch

    def g(fn="nvfp4_grouped_gemm_w4a16", **kw):
        a = dict(a=FAKE, a_rows=64, K=256, lda=256, ridx=FAKE, offs=FAKE, groups=4, rows=128, wc=FAKE,
                 ws=FAKE, wt=FAKE, N=16, c=FAKE, ct=0, ldc=16, stream=None)
        if fn == "mxfp4_grouped_gemm_w4a16":
            del a["wt"]
        a.update(kw)
        return getattr(L, fn)(*a.values())

    for fn in ("nvfp4_grouped_gemm_w4a16", "mxfp4_grouped_gemm_w4a16"):
        assert g(fn, groups=0) == SHAPE
        assert g(fn, groups=(1 << 16) + 1) == SHAPE
        assert g(fn, offs=None) == NULL
        assert g(fn, rows=-1) == SHAPE
        assert g(fn, ridx=None) == SHAPE            # without a gather A needs >= rows rows
        assert g(fn, a_rows=0) == SHAPE
        assert g(fn, K=96, lda=96) == SHAPE
        assert g(fn, ldc=8) == LAYOUT
        assert g(fn, a=None) == NULL
    assert g(K=320, lda=320) != SHAPE                 # NVFP4: K % 64
    assert g("mxfp4_grouped_gemm_w4a16", K=320, lda=320) == SHAPE   # MXFP4: K % 128
    assert g(wt=None) == NULL
    assert L.nvfp4_grouped_gemm_w4a4_workspace(64, 256) == L.gemm_w4a4_workspace(64, 256, 1)

    def q(**kw):
        a = dict(a=FAKE, a_rows=64, K=256, lda=256, ridx=FAKE, offs=FAKE, groups=4, rows=128, wc=FAKE,
                 ws=FAKE, wt=FAKE, N=16, c=FAKE, ct=0, ldc=16, work=FAKE, work_bytes=1 << 20, stream=None)
        a.update(kw)
        return L.nvfp4_grouped_gemm_w4a4(*a.values())

    assert q(work_bytes=100) == WORKSPACE
    assert q(groups=0) == SHAPE
    # the grouped kernel's 2 GiB limits are checked before the quantizer would run
    # (no device here: a limit checked after the launch would report NO_DEVICE)
    big = (1 << 33) // 256                               # A's packed codes of 2^32 bytes
    assert q(a_rows=big, rows=big, ridx=None, work_bytes=1 << 40) == SHAPE
    assert q(N=(1 << 31) // 128, ldc=(1 << 31) // 128) == SHAPE   # one expert's codes of 2 GiB
    assert g(a_rows=1 << 22, lda=256) == SHAPE           # bf16 A of 2 GiB

    def qp(**kw):
        a = dict(ac=FAKE, asc=FAKE, at=FAKE, a_rows=64, K=256, ridx=FAKE, offs=FAKE, groups=4, rows=128,
                 wc=FAKE, ws=FAKE, wt=FAKE, N=16, c=FAKE, ct=0, ldc=16, stream=None)
        a.update(kw)
        return L.nvfp4_grouped_gemm_w4a4_prequant(*a.values())

    assert qp(at=None) == NULL
    assert qp(K=40) == SHAPE
    assert qp(a_rows=big, rows=big, ridx=None) == SHAPE
    if not torch.cuda.is_available():
        assert g() == NO_DEVICE and q() == NO_DEVICE and qp() == NO_DEVICE
    assert g(rows=0, a=None, c=None, wc=None, ws=None, wt=None, ridx=None, a_rows=0) == 0   # empty: no-op
    assert g(rows=0, K=40) == SHAPE and g(rows=0, offs=None) == NULL


def test_python_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    import block_scaled_fp4_04_amd as fp4

    monkeypatch.setattr(fp4, "_lib", None)
    monkeypatch.setattr(fp4, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="no fallback"):
        fp4.lib()


def test_noalloc_validation(L):
    import torch

    def na(**kw):
        a = dict(a=FAKE, M=64, K=256, lda=256, mode=1, wc=FAKE, ws=FAKE, wt=FAKE, N=32, c=FAKE, ct=1, ldc=32,
                 stream=None)
        a.update(kw)
        return L.gemm_w4a4_noalloc(*a.values())

    assert na(a=None) == NULL
    assert na(wt=None) == NULL
    assert na(K=40, lda=40) == SHAPE
    assert na(mode=7) == DTYPE
    assert na(ldc=16) == LAYOUT
    # beyond the 32 MiB scratch: refused on the host, before any device call
    assert na(M=12000, K=5120, lda=5120) == WORKSPACE
    assert na(M=4096, K=16384, lda=16384) == WORKSPACE
    if not torch.cuda.is_available():
        assert na() == NO_DEVICE and na(M=8192, K=5120, lda=5120) == NO_DEVICE


def test_read_ceiling_validation(L):
    """The measurement entry point refuses bad arguments on the host, before any
    device call: null pointers, a size that is zero or not a multiple of 16, a grid
    out of range, a misaligned buffer."""
    import torch

    def rc(buf=FAKE, nbytes=1 << 20, grid=256, sink=FAKE):
        return L.fp4blk_read_ceiling(buf, nbytes, grid, sink, None)

    assert rc(buf=None) == NULL
    assert rc(sink=None) == NULL
    assert rc(nbytes=0) == SHAPE
    assert rc(nbytes=1000) == SHAPE
    assert rc(grid=0) == SHAPE
    assert rc(grid=65536) == SHAPE
    assert rc(buf=FAKE + 8) == LAYOUT
    if not torch.cuda.is_available():
        assert rc() == NO_DEVICE


def test_mxfp4_w4a4_workspace_layout_query(L):
    """mxfp4_gemm_w4a4 keeps A segment-major in its workspace exactly when K is a
    multiple of 128 and both operands' codes stay under 2 GiB (the segment
    kernel's 32-bit offsets); row-major otherwise.  A host-only query."""
    seg = L.mxfp4_gemm_w4a4_a_segment_major
    assert seg(8192, 17408, 5120) == 1
    assert seg(1, 1, 128) == 1
    assert seg(300, 520, 96) == 0                         # K % 128 != 0
    assert seg(300, 520, 1056) == 0
    assert seg((1 << 31) // 64, 16, 128) == 0             # A's codes exactly 2 GiB
    assert seg((1 << 31) // 64 - 1, 16, 128) == 1
    assert seg(16, (1 << 31) // 2560 + 1, 5120) == 0      # W's codes past 2 GiB
    assert seg(16, (1 << 31) // 2560, 5120) == 1
    assert seg(0, 16, 128) == 0 and seg(16, 0, 128) == 0 and seg(16, 16, 0) == 0
