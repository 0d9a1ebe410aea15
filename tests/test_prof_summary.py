"""Host-side checks of the rocprofv3 CSV summaries (no GPU): per-dispatch sums over the
per-XCD counter rows, per-kernel averages, and the copy-kernel calibration of FETCH_SIZE and
WRITE_SIZE."""
import os

import pytest

from rank_recurrent_state_amd import prof_summary as ps


def _write(d, name, header, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, name), "w") as f:
        f.write(",".join(header) + "\n")
        for r in rows:
            f.write(",".join(str(x) for x in r) + "\n")


def test_counters_sum_per_dispatch_and_average_per_kernel(tmp_path, capsys):
    h = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    rows = [(1, "kA", "SQ_WAVES", 4), (1, "kA", "SQ_WAVES", 6), (1, "kA", "SQ_INSTS_VALU", 100),
            (2, "kA", "SQ_WAVES", 10), (2, "kA", "SQ_INSTS_VALU", 300), (3, "kB", "SQ_WAVES", 1)]
    _write(str(tmp_path / "r"), "run_counter_collection.csv", h, rows)
    ps.counters(str(tmp_path))
    out = capsys.readouterr().out.splitlines()
    assert out[0].split()[:3] == ["calls", "SQ_INSTS_VALU", "SQ_WAVES"]
    a = out[1].split()
    assert a[0] == "2" and float(a[1]) == 200.0 and float(a[2]) == 10.0 and a[3] == "kA"
    b = out[2].split()
    assert b[0] == "1" and b[1] == "nan" and float(b[2]) == 1.0 and b[3] == "kB"


def test_pmc_scales_by_the_copy_kernel(tmp_path, capsys):
    h = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    # a 1 MiB copy reads 512 KiB and writes 1024 KiB by the counters: scales 2 and 1
    _write(str(tmp_path / "f"), "run_counter_collection.csv", h,
           [(1, "copyBuffer", "FETCH_SIZE", 256), (1, "copyBuffer", "FETCH_SIZE", 256),
            (2, "kA", "FETCH_SIZE", 10), (3, "kA", "FETCH_SIZE", 30)])
    _write(str(tmp_path / "w"), "run_counter_collection.csv", h,
           [(1, "copyBuffer", "WRITE_SIZE", 1024), (2, "kA", "WRITE_SIZE", 4), (3, "kA", "WRITE_SIZE", 4)])
    ps.pmc(str(tmp_path / "f"), str(tmp_path / "w"), 1 << 20)
    out = capsys.readouterr().out.splitlines()
    assert "scale 2.0000" in out[0] and "scale 1.0000" in out[0]
    ka = next(line.split() for line in out if line.endswith("kA"))
    assert ka[0] == "2" and float(ka[1]) == 20.0 and float(ka[2]) == 4.0
    assert int(ka[3]) == 20 * 1024 * 2 and int(ka[4]) == 4 * 1024


def test_trace_averages_durations(tmp_path, capsys):
    h = ["Kernel_Name", "Start_Timestamp", "End_Timestamp"]
    _write(str(tmp_path / "t"), "run_kernel_trace.csv", h,
           [("kA", 0, 2000), ("kA", 5000, 9000), ("kB", 0, 500)])
    ps.trace(str(tmp_path))
    out = capsys.readouterr().out.splitlines()
    a = out[1].split()
    assert a[0] == "2" and float(a[1]) == pytest.approx(3.0) and a[-1] == "kA"


def test_missing_output_is_an_error(tmp_path):
    with pytest.raises(SystemExit):
        ps.counters(str(tmp_path))
