"""Host-side pieces of bench.py that need no GPU: the profile summaries
(rocprofv3 kernel-trace and counter CSVs grouped by kernel and grid) and
the refusal of more than one GPU."""
import csv
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _write(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def test_trace_summary_groups_by_kernel_and_grid(tmp_path, capsys):
    rows = []
    # two whole-layer launches of 100 us and 16 chunked ones of 10 us each
    for i in range(2):
        rows.append(dict(Kernel_Name="attend", Grid_Size_X=1024, Grid_Size_Y=1, Grid_Size_Z=1,
                         Start_Timestamp=1000 * i * 1000, End_Timestamp=1000 * i * 1000 + 100000))
    for i in range(16):
        rows.append(dict(Kernel_Name="attend", Grid_Size_X=64, Grid_Size_Y=1, Grid_Size_Z=1,
                         Start_Timestamp=5000000 + i * 20000, End_Timestamp=5000000 + i * 20000 + 10000))
    p = tmp_path / "run_kernel_trace.csv"
    _write(p, rows)
    bench.trace_summary(str(p))
    out = capsys.readouterr().out.splitlines()
    got = {(l.split()[0], l.split()[1]): (int(l.split()[2]), float(l.split()[4])) for l in out[1:]}
    assert got[("attend", "1024x1x1")] == (2, 100.0)
    assert got[("attend", "64x1x1")] == (16, 10.0)
    # ordered by total time: the 200 us group first
    assert out[1].split()[1] == "1024x1x1"


def test_counter_summary_mean_per_dispatch(tmp_path, capsys):
    rows = []
    # dispatch 1 reports its counter in two rows (summed), dispatch 2 in one
    for d, v in ((1, 10.0), (1, 30.0), (2, 60.0)):
        rows.append(dict(Dispatch_Id=d, Kernel_Name="k", Grid_Size=256, Counter_Name="FETCH_SIZE",
                         Counter_Value=v))
    p = tmp_path / "run_counter_collection.csv"
    _write(p, rows)
    bench.trace_summary(str(p))
    out = capsys.readouterr().out.splitlines()
    f = out[1].split()
    assert f[0] == "k" and f[1] == "256" and int(f[2]) == 2 and f[3] == "FETCH_SIZE"
    assert float(f[4]) == 50.0  # (10 + 30 + 60) / 2 dispatches


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
