"""Host-side checks of the benchmark script (no GPU): it refuses more than one
GPU with a JSON error line, and the HBM traffic it reports comes from a counter
summary only while the kernel sources hash to the value recorded there."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


@pytest.fixture()
def bench_module():
    import bench
    return bench


def _write_summary(path, sha, traffic):
    with open(path, "w") as f:
        f.write("HBM traffic summary\n")
        f.write(f"source_sha256: {sha}\n")
        f.write(f"traffic_bytes_per_dispatch: {traffic}\n")


def test_measured_traffic_follows_the_source_hash(bench_module, tmp_path, monkeypatch):
    b = bench_module
    (tmp_path / "profiles").mkdir()
    src = tmp_path / "k.hip"
    src.write_text("kernel source, first version\n")
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    sha = b.code_sha256(["k.hip"])
    path = tmp_path / "profiles" / "kern.work.hbm_traffic.txt"
    assert b.measured_traffic("kern", "work", ["k.hip"]) is None          # no summary
    _write_summary(path, sha, "151788556.0")
    assert b.measured_traffic("kern", "work", ["k.hip"]) == 151788556
    src.write_text("kernel source, changed\n")                              # counters are stale now
    assert b.measured_traffic("kern", "work", ["k.hip"]) is None


def test_committed_decode_summaries_name_their_source_hash(bench_module):
    """Every committed decode traffic summary records a source hash and a byte
    count (whether they still match is decided at run time)."""
    b = bench_module
    for wl in ("decode_8b", "decode_70b_32k"):
        path = os.path.join(ROOT, "profiles", f"decode_bf16_kernel.{wl}.hbm_traffic.txt")
        text = open(path).read()
        assert "source_sha256:" in text and "traffic_bytes_per_dispatch:" in text
        assert wl in b.DECODE_WORKLOADS


def test_every_profile_summary_names_its_command_and_source():
    """Each committed rocprofv3 summary gives the command that made it (bench.py
    runs only) and, for the library's own kernels, the hash of their device
    code at the time."""
    d = os.path.join(ROOT, "profiles")
    names = sorted(os.listdir(d))
    assert names
    for name in names:
        text = open(os.path.join(d, name)).read()
        assert "Command (from the repository root" in text, name
        assert "python3 bench.py" in text and "_work" not in text, name
        if name.split(".")[0].startswith(("decode_bf16_kernel", "prefill_bf16_kernel", "calib_tiled_kernel",
                                         "mkc_values_bf16_kernel")):
            assert "source_sha256:" in text, name
