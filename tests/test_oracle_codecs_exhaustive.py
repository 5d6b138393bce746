"""Exhaustive pins of the oracle's element encoders (CPU only, about 30 s on 8 cores).

tests/native/codec_exhaustive.c checks the oracle's E2M1 encoder on every non-NaN
fp32 bit pattern and its E4M3 encoder on every non-negative one against a
brute-force nearest-value search written independently of the oracle (decoded
candidates, fp64 distances, even tie-break, saturation).  A copy of the oracle
with one tie rule flipped must fail the same check, so the check can see the
kind of mistake it is there for.
"""
import os
import shutil
import subprocess

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "native", "codec_exhaustive.c")


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("no C compiler")
    out = str(tmp_path_factory.mktemp("codecx") / "codec_exhaustive")
    subprocess.run([cc, "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", SRC, "-o", out, "-ldl", "-lm"],
                   check=True)
    return out


def test_encoders_match_brute_force_on_every_pattern(exe):
    r = subprocess.run([exe, oracle.build(force=False)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "E2M1: 4278190082 patterns, 0 mismatches" in r.stdout, r.stdout
    assert "E4M3: 2139095041 patterns, 0 mismatches" in r.stdout, r.stdout


def test_the_check_sees_a_flipped_tie(exe, tmp_path):
    """The oracle with the tie at 0.25 sent to 0.5 instead of 0 (the even code):
    exactly the two patterns +-0.25 must be reported."""
    src = open(oracle._SRC).read()
    bad = src.replace("if (a <= 0.25)      m = 0;", "if (a < 0.25)       m = 0;")
    assert bad != src
    p = tmp_path / "mutant.c"
    p.write_text(bad)
    lib = str(tmp_path / "libmutant.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", str(p),
                    "-o", lib, "-lm"], check=True)
    r = subprocess.run([exe, lib, "e2m1"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 1, r.stdout + r.stderr
    assert "E2M1: 4278190082 patterns, 2 mismatches" in r.stdout, r.stdout
