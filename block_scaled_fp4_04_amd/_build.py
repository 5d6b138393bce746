"""Build libfp4blk.so (HIP, gfx950) in-tree with hipcc.

The library links against the HIP runtime that torch ships, so a stream handle
taken from torch (``torch.cuda.current_stream().cuda_stream``) is valid inside
the library: one process must not carry two HIP runtimes.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "libfp4blk.so")
SOURCES = ["abi.hip", "quant.hip", "gemm_nv.hip", "gemv_nv.hip", "gemm_mx.hip", "measure.hip"]
HEADERS = ["device_common.h", "internal.h"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _torch_libdir() -> str:
    import importlib.util

    spec = importlib.util.find_spec("torch")
    if spec is None or not spec.submodule_search_locations:
        raise RuntimeError("torch is required to locate its HIP runtime")
    return os.path.join(list(spec.submodule_search_locations)[0], "lib")


def flags():
    return [
        "--offload-arch=gfx950",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        # IEEE fp32 division for the quantizers; no fast-math anywhere
        "-fhip-fp32-correctly-rounded-divide-sqrt",
        "-fno-fast-math",
        # keep the compiler from forming packed fp32 arithmetic
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall",
        "-Wno-unused-function",
        f"-I{INCLUDE}",
        f"-I{CSRC}",
    ]


def _compile(src: str, verbose: bool) -> tuple[str, subprocess.CompletedProcess]:
    obj = os.path.join(LIBDIR, src.replace(".hip", ".o"))
    cmd = [HIPCC, *flags(), "-c", os.path.join(CSRC, src), "-o", obj]
    cmd.remove("-shared")
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    return obj, subprocess.run(cmd, capture_output=True, text=True)


def build(verbose: bool = False) -> str:
    """Compile every HIP source into LIB (the sources in parallel); always recompiles."""
    from concurrent.futures import ThreadPoolExecutor

    os.makedirs(LIBDIR, exist_ok=True)
    tlib = _torch_libdir()
    jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    objs = []
    for src, (obj, r) in zip(SOURCES, results):
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError(f"hipcc failed on {src}")
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp,
           f"-L{tlib}", f"-Wl,-rpath,{tlib}", "-Wl,--no-undefined", "-lamdhip64"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc link failed")
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
