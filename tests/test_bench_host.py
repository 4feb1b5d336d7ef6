"""Host-side logic of bench.py (no GPU): the one-GPU guard, the algorithmic byte
and VALU-operation models at the kodak768 shape, and the reading of committed
counter summaries (used only while their kernel-source hash matches)."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_byte_and_op_models_at_kodak768():
    P, N, M = 768 * 512, 50_000, 4
    b = bench.algorithmic_bytes(P, N)
    # compulsory bytes per call: propagate 64 P + 24 N, forward 44 P + 40 N,
    # backward 44 P + 84 N, Adam 324 N; a step is 152 P + 472 N
    assert b["fwd_bwd"] == 88 * P + 124 * N
    assert b["propagate"] == 64 * P + 24 * N
    assert b["adam"] == 324 * N
    assert b["fwd"] == 44 * P + 40 * N
    assert b["propagate"] + b["fwd_bwd"] + b["adam"] == bench.step_bytes(P, N) == 152 * P + 472 * N
    # 83.4 MB per kodak768 iteration, 699.4 MB per img2048 iteration
    assert abs(bench.step_bytes(P, N) / 1e6 - 83.37) < 0.01
    assert abs(bench.step_bytes(2048 * 2048, 131_072) / 1e6 - 699.4) < 0.1
    o = bench.algorithmic_ops(P, N, M)
    assert o["propagate"] == P * 44 * 30
    assert o["fwd_bwd"] == P * 650
    assert o["fwd"] == P * 164 and o["adam"] == N * 120
    assert abs(bench.VALU_PEAK_TOPS - 39.3216) < 1e-9


def test_profile_rows_and_source_gate(tmp_path, monkeypatch):
    f = tmp_path / "x.txt"
    f.write_text("header\nsource_sha256: abc\ntraffic kernel=k_a bytes_per_launch=12 fetch=5 write=7\n"
                 "valu kernel=k_a issue_frac=0.5 insts_per_wave=10.0 us=1.0\n")
    digest, rows = bench._profile_rows(str(f), "traffic")
    assert digest == "abc" and rows["k_a"]["bytes_per_launch"] == "12"
    digest, rows = bench._profile_rows(str(f), "valu")
    assert rows["k_a"]["issue_frac"] == "0.5"
    assert bench._profile_rows(str(tmp_path / "missing.txt"), "valu") == (None, {})
    # the committed summaries are used only for the kernel source they were taken on
    monkeypatch.setattr(bench, "source_digest", lambda: "not-the-hash")
    assert bench.measured_traffic("kodak768", "fwd_bwd") is None
    assert bench.measured_valu_issue("kodak768", "fwd_bwd") is None
