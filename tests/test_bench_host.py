"""Host-side logic of bench.py (no GPU): the one-GPU guard, the byte model
of a replay-decode step, and the arithmetic that turns rocprofv3 counter
files into HBM traffic (calibrated by a plain copy of known size)."""
import csv
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
from exact_replay_decode_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def write_counters(path, counter, rows):
    """rows: (dispatch id, kernel name, value) -> a counter-collection CSV."""
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for d, name, v in rows:
            w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": v})


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_replay_step_bytes_by_hand():
    """Two slots with k = 0 and k = 3 at Q = 4 (the second fills its chunk),
    H=2, G=1, P=4, N=8, bf16 everything: sum the pieces by hand."""
    H, G, P, N, Q = 2, 1, 4, 8, 4
    state_bf = H * P * N * 2                   # bf16 read copy
    new_tok = H * P * 2 + H * 2 + 2 * G * N * 2
    append = H * P * 2 + H * 2 + G * N * 2
    y = H * P * 2
    per_row = H * P * 2 + G * N * 2 + H * 2    # buffered x, B, raw dt
    commit = H * P * N * (4 + 4 + 2) + Q * per_row
    want = 2 * (state_bf + new_tok + append + y) + 3 * per_row + commit
    assert bench.replay_step_bytes([0, 3], Q, H, G, P, N) == want


def test_prefill_traffic_from_counters(tmp_path):
    copy_kib = bench.CALIB_BYTES / 1024
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    # the copy's FETCH_SIZE reads half its bytes (factor 2), WRITE_SIZE all
    write_counters(f, "FETCH_SIZE", [(1, "copyBuffer", copy_kib / 2),
                                     (2, bench.PREFILL_KERNEL + "(args)", 1000.0),
                                     (3, bench.PREFILL_KERNEL + "(args)", 3000.0)])
    write_counters(w, "WRITE_SIZE", [(1, "copyBuffer", copy_kib),
                                     (2, bench.PREFILL_KERNEL + "(args)", 500.0),
                                     (3, bench.PREFILL_KERNEL + "(args)", 500.0)])
    rec = bench.write_traffic(str(f), str(w), [], out=str(tmp_path / "t.json"))
    assert rec["copy_calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert rec["copy_calibration"]["write_factor"] == pytest.approx(1.0)
    assert rec["traffic_bytes_per_launch"] == pytest.approx(1024 * (2000.0 * 2 + 500.0))


def test_decode_traffic_matches_algorithmic_bytes(tmp_path):
    """Counter values built from the exact bytes of each dispatch's buffer
    fills give a ratio of 1; a different dispatch count in the two files is
    refused."""
    S, H, G, P, N, Q = 256, 32, 1, 64, 128, 256
    n = 40
    k0 = synth.replay_prefix_lengths(S, Q, 1) % Q
    alg = [bench.replay_step_bytes((k0 + i) % Q, Q, H, G, P, N) for i in range(n)]
    copy_kib = bench.CALIB_BYTES / 1024
    name = bench.DECODE_KERNEL + "(ssd::DecodeArgs)"
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    # all of a dispatch's bytes in FETCH_SIZE (calibration factor 2)
    write_counters(f, "FETCH_SIZE", [(0, "copyBuffer", copy_kib / 2)] +
                   [(i + 1, name, a / 1024 / 2) for i, a in enumerate(alg)])
    write_counters(w, "WRITE_SIZE", [(0, "copyBuffer", copy_kib)] +
                   [(i + 1, name, 0.0) for i in range(n)])
    rec = bench.write_decode_traffic(str(f), str(w), [], out=str(tmp_path / "d.json"))
    assert rec["dispatches"] == n
    assert rec["traffic_over_algorithmic"] == pytest.approx(1.0, rel=1e-12)
    assert rec["algorithmic_bytes_per_dispatch_mean"] == pytest.approx(np.mean(alg))
    write_counters(w, "WRITE_SIZE", [(0, "copyBuffer", copy_kib)] +
                   [(i + 1, name, 0.0) for i in range(n - 1)])
    with pytest.raises(SystemExit):
        bench.write_decode_traffic(str(f), str(w), [], out=str(tmp_path / "d2.json"))
