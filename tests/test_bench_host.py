"""Host-side checks of bench.py (no GPU): the one-GPU rule, the algorithmic byte
count of the decode step, and the source-hash guard on the committed HBM traffic
figure."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_decode_bytes_are_the_algorithmic_bytes():
    # A bf16 [M][K] + W codes [N][K/2] + E4M3 bytes [N][K/16] + fp32 tensor scale + bf16 C [M][N]
    for M in (1, 4, 16):
        assert bench.decode_bytes(M) == M * 5120 * 2 + 17408 * 2560 + 17408 * 320 + 4 + M * 17408 * 2
    assert bench.decode_bytes(1) == 50180100


def test_traffic_is_reported_only_while_the_kernel_sources_match(tmp_path, monkeypatch):
    d = json.load(open(bench.TRAFFIC_JSON))
    got = bench.measured_traffic((1, 4, 16))
    if got is not None:  # the committed figure belongs to the committed sources
        per = d["per_M_bytes"]
        assert got == round(sum(per[m]["fetch"] + per[m]["write"] for m in ("1", "4", "16")) / 3)
    stale = dict(d, sha256="0" * 64)
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps(stale))
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(p))
    assert bench.measured_traffic((1, 4, 16)) is None


def test_component_groups_are_the_only_choices():
    assert bench.COMPONENT_GROUPS == ["quant", "prefill_m4096", "mxfp4_w4a16", "m8192", "moe"]
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--only", "nope"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0 and "invalid choice" in r.stderr
