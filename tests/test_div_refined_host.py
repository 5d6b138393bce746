"""Host check of the shared-divisor division the NVFP4 quantizers use (CPU only).

The quantizer kernels divide the 16 values of a block by one step d with gfx950's
own correctly rounded division sequence, its reciprocal computed once per block
(csrc/quant.hip, rcp_refined / div_refined).  tests/native/div_refined_check.c
replays that sequence with C's fmaf for every reciprocal within one ulp of 1/d
(the accuracy the hardware reciprocal guarantees), on random quotients, on
quotients next to every E2M1 grid point and midpoint and every E4M3 rounding
boundary, and next to fp32 rounding midpoints, and compares each result with the
IEEE division a / d.  This pins the arithmetic identity the kernels rely on; the
GPU tests then check the kernels' bytes against the oracle.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "native", "div_refined_check.c")


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    out = str(tmp_path_factory.mktemp("divchk") / "div_refined_check")
    subprocess.run([cc, "-O2", "-ffp-contract=off", "-fno-fast-math", SRC, "-o", out, "-lm"], check=True)
    return out


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_shared_reciprocal_division_is_correctly_rounded(exe, seed):
    r = subprocess.run([exe, str(seed), "1500", "1500"], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert " 0 mismatches" in r.stdout, r.stdout


def test_the_check_sees_a_weaker_sequence(exe, tmp_path):
    """The same program with the corrections removed (q = a y alone) must fail:
    the check is able to tell a correctly rounded quotient from an approximate one."""
    src = open(SRC).read().replace("volatile float q0 = a * y;", "volatile float q0 = a * y;\n    return q0;")
    p = tmp_path / "weak.c"
    p.write_text(src)
    out = str(tmp_path / "weak")
    subprocess.run([shutil.which("gcc") or "cc", "-O2", "-ffp-contract=off", str(p), "-o", out, "-lm"], check=True)
    r = subprocess.run([out, "1", "200", "200"], capture_output=True, text=True)
    assert r.returncode == 1 and " 0 mismatches" not in r.stdout
