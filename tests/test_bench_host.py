"""Host-side pieces of bench.py (no GPU): the algorithmic byte counts the roofline is
priced on, the one-GPU guard, and the HBM-traffic summary built from counter CSVs.

The expected byte counts are written out from the layout of the packed grid (4-bit
codes, one fp16 scale and one 4-bit zero per group of 128 along K, bf16 X and Y) at
the decode, lm_head and prefill shapes, not taken from bench.py."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _layout_bytes(M, N, K, y_bytes):
    groups = K // 128
    codes = N * K // 2          # 8 codes per uint32
    scales = N * groups * 2     # fp16
    zeros = N * groups // 2     # 8 zeros per uint32
    return codes + scales + zeros + 2 * M * K + y_bytes * M * N


@pytest.mark.parametrize("M,N,K,expected", [
    (1, 9728, 2560, 12_962_816),   # decode gate/up
    (1, 2560, 9728, 12_962_816),   # decode down
    (1, 512, 512, 138_240),        # single 512 x 512
    (8192, 9728, 2560, 214_264_832),  # prefill gate/up
])
def test_algo_bytes_linear(M, N, K, expected):
    assert _layout_bytes(M, N, K, 2) == expected
    assert bench.algo_bytes(M, N, K) == expected


def test_algo_bytes_lmhead_writes_no_logits():
    # 16 rows against the 151936-column vocabulary: weights and X, plus 16 draft ids in,
    # 16 argmax ids and one accepted length out
    expected = _layout_bytes(16, 151936, 2560, 0) + 16 * 4 + 16 * 4 + 4
    assert expected == 202_156_932
    assert bench.algo_bytes(16, 151936, 2560, lmhead=True) == expected


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _counter_csv(path, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for k, c, v in rows:
            w.writerow({"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_pmc_summary_scales_by_the_copy_calibration(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path / "out"))
    algo = bench.algo_bytes(1, 9728, 2560)
    calib = bench.CALIB_BYTES
    # the copy reads half its source bytes in FETCH_SIZE and all of them in WRITE_SIZE
    _counter_csv(tmp_path / "cf.csv", [("copy_kernel", "FETCH_SIZE", calib / 2 / 1024)])
    _counter_csv(tmp_path / "cw.csv", [("copy_kernel", "WRITE_SIZE", calib / 1024)])
    # two dispatches per counter whose scaled mean is 1.1x the algorithmic fetch, and
    # the output's bytes written
    f_kib = 1.1 * algo / 2 / 1024
    _counter_csv(tmp_path / "f.csv", [("gemv_kernel<8, 8, true>", "FETCH_SIZE", f_kib * 0.9),
                                      ("gemv_kernel<8, 8, true>", "FETCH_SIZE", f_kib * 1.1),
                                      ("prep_kernel", "FETCH_SIZE", 1e9)])
    _counter_csv(tmp_path / "w.csv", [("gemv_kernel<8, 8, true>", "WRITE_SIZE", 0.0),
                                      ("gemv_kernel<8, 8, true>", "WRITE_SIZE", 0.0)])
    bench.pmc_summary("decode_gemv_m1", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                      str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv"), commands=["cmd"])
    text = open(tmp_path / "out" / "gemv_kernel__decode_gemv_m1__pmc.txt").read()
    fields = dict(l.split(": ", 1) for l in text.splitlines() if not l.startswith("#"))
    assert int(fields["fetch_dispatches"]) == 2
    assert float(fields["hbm_fetch_bytes_per_launch"]) == pytest.approx(1.1 * algo, rel=1e-6)
    assert float(fields["algorithmic_bytes_per_launch"]) == algo
    assert float(fields["traffic_over_algorithmic"]) == pytest.approx(1.1, abs=1e-4)
    assert fields["kernel_source_sha"] == bench.kernel_source_sha("gemv_kernel")
