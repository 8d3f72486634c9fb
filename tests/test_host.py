"""Host-side logic of the benchmark (no GPU): the one-GPU refusal, the code
digest that keys the committed HBM traffic records, and those records'
arithmetic."""
import glob
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_code_digest_ignores_comments_and_layout_only():
    a = b"int f(int x) {\n  return x + 1;  // one more\n}\n"
    b = b"/* the successor */ int f(int x)\n{ return x + 1; }"
    c = b"int f(int x) { return x + 2; }"
    assert bench.code_digest(a) == bench.code_digest(b)
    assert bench.code_digest(a) != bench.code_digest(c)


def test_kernel_code_digest_follows_local_includes(tmp_path, monkeypatch):
    csrc = tmp_path / "scaled_quantization_amd" / "csrc"
    inc = tmp_path / "include"
    csrc.mkdir(parents=True)
    inc.mkdir()
    (csrc / "k.hip").write_bytes(b'#include "h.hpp"\n#include <hip/hip_runtime.h>\nint k;\n')
    (csrc / "h.hpp").write_bytes(b'#include "api.h"\nint h;\n')
    (inc / "api.h").write_bytes(b"int api;\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    d0 = bench.kernel_code_digest("k.hip")
    (inc / "api.h").write_bytes(b"int api; // a comment\n")
    assert bench.kernel_code_digest("k.hip") == d0
    (inc / "api.h").write_bytes(b"int api2;\n")
    assert bench.kernel_code_digest("k.hip") != d0


def test_measured_traffic_only_for_the_recorded_code(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    (tmp_path / "scaled_quantization_amd" / "csrc").mkdir(parents=True)
    (tmp_path / "scaled_quantization_amd" / "csrc" / "k.hip").write_bytes(b"int k;\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    rec = {"kernel_code_sha256": bench.kernel_code_digest("k.hip"), "bytes_per_launch": 123}
    (tmp_path / "profiles" / "x_traffic.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("x", "k.hip") == 123
    (tmp_path / "scaled_quantization_amd" / "csrc" / "k.hip").write_bytes(b"int k2;\n")
    assert bench.measured_traffic("x", "k.hip") is None
    assert bench.measured_traffic("absent", "k.hip") is None


@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(ROOT, "profiles", "*_traffic.json"))))
def test_traffic_record_arithmetic(path):
    r = json.load(open(path))
    c = r["copy_reference"]
    # the copy kernel's counters calibrate the factors: bytes moved / counter KiB
    assert abs(c["fetch_factor"] - c["bytes_read"] / (c["fetch_size_kib"] * 1024)) < 1e-4
    assert abs(c["write_factor"] - c["bytes_written"] / (c["write_size_kib"] * 1024)) < 1e-4
    fb = r["fetch_size_kib_per_dispatch"] * 1024 * c["fetch_factor"]
    wb = r["write_size_kib_per_dispatch"] * 1024 * c["write_factor"]
    assert abs(fb - r["fetch_bytes_per_launch"]) / fb < 1e-3
    assert abs(wb - r["write_bytes_per_launch"]) / wb < 1e-3
    assert r["bytes_per_launch"] == r["fetch_bytes_per_launch"] + r["write_bytes_per_launch"]
    assert abs(r["ratio_to_algorithmic"] - r["bytes_per_launch"] / r["algorithmic_bytes_per_launch"]) < 1e-3
    # no kernel moves less than its algorithmic bytes
    assert r["ratio_to_algorithmic"] > 0.99


def test_every_only_mode_has_its_own_launch():
    # bench.py --only <mode> launches one kernel for counter runs; a mode
    # without a branch of its own in kernel_only would stop with an error
    import re
    src = open(os.path.join(ROOT, "bench.py")).read()
    choices = re.search(r'"--only", choices=\(([^)]*)\)', src).group(1)
    modes = [c.strip().strip('"') for c in choices.replace("\n", "").split(",") if c.strip()]
    body = src[src.index("def kernel_only"):src.index("_COPY = []")]
    assert len(modes) >= 12
    for m in modes:
        assert f'args.only == "{m}"' in body or re.search(rf'args\.only in \([^)]*"{m}"', body), m
