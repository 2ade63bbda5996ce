"""CPU tests of bench.py's host logic: the byte-counter summary (each counter
scaled by what it reads for plain kernels of known traffic), the rule that a
committed counter summary is used only while the expert kernels' sources are
unchanged, and the one-GPU guard.
"""
import csv
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _counter_csv(path, rows):
    """rocprofv3-style counter_collection CSV: one row per (dispatch, counter instance)."""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for disp, name, counter, val in rows:
            w.writerow(dict(Dispatch_Id=disp, Kernel_Name=name, Counter_Name=counter, Counter_Value=val))


def test_pmc_summary_scales_each_counter_by_its_calibration(tmp_path, capsys):
    kib = bench.CAL_BYTES / 1024
    # the calibration kernels read half of the true bytes on FETCH_SIZE and all of them on WRITE_SIZE
    _counter_csv(tmp_path / "cf.csv", [(1, "k_read(...)", "FETCH_SIZE", kib / 4), (1, "k_read(...)", "FETCH_SIZE", kib / 4),
                                       (2, "k_copy(...)", "FETCH_SIZE", 2 * kib)])
    _counter_csv(tmp_path / "cw.csv", [(1, "k_read(...)", "WRITE_SIZE", 0.0), (2, "k_copy(...)", "WRITE_SIZE", kib)])
    # two launches of the GEMV: 1000 and 3000 KiB fetched (several counter instances per dispatch add up),
    # 10 KiB written each
    _counter_csv(tmp_path / "f.csv", [(5, "void moe::k_gateup_gemv<2>(moe::ExpertArgs)", "FETCH_SIZE", 600.0),
                                      (5, "void moe::k_gateup_gemv<2>(moe::ExpertArgs)", "FETCH_SIZE", 400.0),
                                      (9, "void moe::k_gateup_gemv<2>(moe::ExpertArgs)", "FETCH_SIZE", 3000.0),
                                      (7, "moe::k_combine(...)", "FETCH_SIZE", 8.0)])
    _counter_csv(tmp_path / "w.csv", [(5, "void moe::k_gateup_gemv<2>(moe::ExpertArgs)", "WRITE_SIZE", 10.0),
                                      (9, "void moe::k_gateup_gemv<2>(moe::ExpertArgs)", "WRITE_SIZE", 10.0),
                                      (7, "moe::k_combine(...)", "WRITE_SIZE", 4.0)])
    bench.pmc_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(tmp_path / "cf.csv"),
                      str(tmp_path / "cw.csv"))
    out = capsys.readouterr().out
    assert "factor 2.0000" in out and "factor 1.0000" in out
    lines = [l for l in out.splitlines() if l.startswith("traffic k_gateup_gemv")]
    assert len(lines) == 1
    # mean fetch 2000 KiB x 2 (calibrated) + mean write 10 KiB x 1
    assert float(lines[0].split()[3]) == pytest.approx((2000 * 2 + 10) * 1024, rel=1e-6)
    assert f"source_sha256 {bench.source_sha256()}" in out


def test_traffic_only_while_the_kernel_sources_match(monkeypatch):
    path = os.path.join(ROOT, "profiles", "k_gateup_gemv_decode32_pmc.md")
    with open(path) as f:
        sha = [ln.split()[1] for ln in f if ln.startswith("source_sha256 ")]
    t = bench.traffic_of("k_gateup_gemv", "decode32")
    if sha and sha[0] == bench.source_sha256():
        assert t is not None and 1e9 < t < 3e9  # the committed summary of the decode-32 GEMV
    else:
        assert t is None  # taken on other kernel sources: not reported
    monkeypatch.setattr(bench, "source_sha256", lambda: "0" * 64)
    assert bench.traffic_of("k_gateup_gemv", "decode32") is None
    assert bench.traffic_of("k_gateup_gemv", "no_such_workload") is None


def test_source_hash_covers_the_expert_kernel_sources():
    names = sorted(os.path.basename(p) for p in bench.KERNEL_SRC)
    assert names == ["k_expert.hip", "moe_internal.h"]
    assert all(os.path.exists(p) for p in bench.KERNEL_SRC)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
