"""Host-side logic of bench.py: the one-GPU guard, the kernel-source hash
that ties a committed counter summary to the code it was taken on, and the
algorithmic work it reports (4*|I|*|J|*D flop per kept block pair)."""

import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_kernel_hash_follows_code_not_comments(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(src)])
    src.write_text("int f(int x) { return x + 1; }\n")
    h0 = bench.kernel_hash()
    src.write_text("// a comment\nint f(int x)   {\n  /* block\n comment */ return x + 1;  // tail\n}\n")
    assert bench.kernel_hash() == h0
    src.write_text("int f(int x) { return x + 2; }\n")
    assert bench.kernel_hash() != h0


def test_kept_flops_counts_ragged_blocks():
    # N = 100 tokens, block 64: blocks of 64 and 36 tokens; D = 8
    count = np.array([[[1, 2]]], np.int32)
    idx = np.array([[[[1, 0], [0, 1]]]], np.int32)
    # (I0, J1) 64*36, (I1, J0) 36*64, (I1, J1) 36*36
    expect = 4.0 * (64 * 36 + 36 * 64 + 36 * 36) * 8
    assert bench.kept_flops(count, idx, 100, 64, 8) == expect
    # every pair kept: the dense count
    full = np.array([[[2, 2]]], np.int32)
    both = np.array([[[[0, 1], [0, 1]]]], np.int32)
    assert bench.kept_flops(full, both, 100, 64, 8) == bench.dense_flops(1, 1, 100, 8)


def test_select_floor_from_counted_instructions():
    """The selection's compute floor: rows x counted VALU instructions per
    row x 4 cycles over 1024 SIMDs at 2.4 GHz, for the row's sort size, and
    only while the counter summary matches the kernel's sources."""
    import json
    with open(bench.SELECT_COUNTERS_FILE) as fh:
        rec = json.load(fh)
    if rec["kernel_sha"] != bench.kernel_hash(bench.SELECT_SOURCES):
        assert bench.select_floor_ms(20480, 512) is None
        return
    per_row = rec["valu_instructions_per_row"]["512"]
    want = 20480 * per_row * 4 / 1024 / 2.4e9 * 1e3
    assert abs(bench.select_floor_ms(20480, 512) - want) < 1e-12
    assert abs(bench.select_floor_ms(20480, 278) - want) < 1e-12     # sort size 512 too
    assert bench.select_floor_ms(100, 929) == 100 * rec["valu_instructions_per_row"]["1024"] \
        * 4 / 1024 / 2.4e9 * 1e3
    assert bench.select_floor_ms(100, 100) is None                  # size 128 not counted


def test_sustained_clock_is_tied_to_the_kernel_source(tmp_path, monkeypatch):
    import json
    rec = {"kernel_sha": bench.kernel_hash(), "nominal_ghz": 2.4,
           "workloads": {"w": {"ghz": 1.8, "boxes": []}}}
    path = tmp_path / "clock.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "CLOCK_FILE", str(path))
    got = bench.read_sustained_clock("w", 1125.0)
    # peak at 1.8 GHz = 2500 * 1.8 / 2.4 = 1875 TFLOP/s
    assert got["ghz"] == 1.8 and got["peak_at_clock"] == 1875.0
    assert got["frac_at_clock"] == 0.6
    assert bench.read_sustained_clock("other", 1125.0) is None
    rec["kernel_sha"] = "0" * 16
    path.write_text(json.dumps(rec))
    assert bench.read_sustained_clock("w", 1125.0) is None
