"""Host logic of bench.py (CPU only): when the rocprofv3 counter passes start,
the multi-GPU refusal, and the parsers of the counter files.

The counter passes are child processes; they must never start from a process
that itself runs under the profiler (its GPU is already initialised there) nor
from the plain-copy calibration run.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


class _Started(Exception):
    pass


@pytest.fixture()
def passes(monkeypatch):
    calls = []

    def fake(workload, dtype, outroot, timeout_s=170):
        calls.append(workload)
        raise _Started()
    monkeypatch.setattr(bench, "run_counter_passes", fake)
    for k in list(os.environ):
        if k.startswith("ROCPROF_"):
            monkeypatch.delenv(k)
    return calls


def _run(argv):
    """main() up to the first GPU use: on this host it stops at the GPU check."""
    try:
        bench.main(argv)
    except _Started:
        return "counters"
    except AssertionError as e:
        assert "GPU" in str(e)
        return "gpu"
    return "returned"


def test_default_run_starts_counter_passes_on_the_headline(passes, tmp_path):
    assert _run(["--counters-dir", str(tmp_path)]) == "counters"
    assert passes == [bench.HEADLINE]


def test_single_workload_counters_only_when_asked(passes, tmp_path):
    assert _run(["--workload", "c3", "--no-cpu-baseline"]) == "gpu"
    assert _run(["--workload", "c3", "--counters", "--counters-dir", str(tmp_path)]) == "counters"
    assert passes == ["c3"]


def test_no_counters_flag(passes):
    assert _run(["--no-counters"]) == "gpu"
    assert passes == []


def test_copy_calibration_never_starts_passes(passes):
    assert _run(["--copy-calibration", "8"]) == "gpu"
    assert passes == []


def test_not_nested_under_the_profiler(passes, monkeypatch):
    monkeypatch.setenv("ROCPROF_OUTPUT_PATH", "/tmp/x")
    assert _run([]) == "gpu"
    assert _run(["--workload", "c4", "--counters"]) == "gpu"
    assert passes == []


def test_counter_child_and_other_ops_skip_passes(passes):
    assert _run(["--counter-child", "--workload", "c4"]) == "gpu"
    assert _run(["--op", "append"]) == "gpu"
    assert _run(["--op", "padded", "--counters"]) == "gpu"
    assert passes == []


def test_more_than_one_gpu_exits(passes, capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err
    assert passes == []


def test_counter_csv_parser(tmp_path):
    p = tmp_path / "run_counter_collection.csv"
    hdr = "Correlation_Id,Dispatch_Id,Agent_Id,Queue_Id,Process_Id,Thread_Id,Grid_Size,Kernel_Id,Kernel_Name," \
          "Workgroup_Size,LDS_Block_Size,Scratch_Size,VGPR_Count,Accum_VGPR_Count,SGPR_Count,Counter_Name," \
          "Counter_Value,Start_Timestamp,End_Timestamp\n"
    rows = []
    for i, (name, val) in enumerate([("GRBM_GUI_ACTIVE", 800.0), ("SQ_WAVE_CYCLES", 5.0),
                                     ("GRBM_GUI_ACTIVE", 1600.0), ("SQ_WAVE_CYCLES", 7.0)]):
        disp = 1 + i // 2
        rows.append("%d,%d,1,1,1,1,64,3,\"k<a, b>(p)\",64,0,0,8,0,16,%s,%r,%d,%d\n"
                    % (disp, disp, name, val, 1000 * disp, 1000 * disp + 500))
    p.write_text(hdr + "".join(rows))
    vals, durs = bench.parse_counter_csv(str(p))
    assert list(vals) == ["k<a, b>(p)"]
    assert vals["k<a, b>(p)"]["GRBM_GUI_ACTIVE"] == [800.0, 1600.0]
    assert vals["k<a, b>(p)"]["SQ_WAVE_CYCLES"] == [5.0, 7.0]
    assert durs["k<a, b>(p)"] == [500.0, 500.0]
    # the first dispatch (cold caches, first launch) is left out when there are more
    assert bench._mean_tail([800.0, 1600.0, 2400.0]) == 2000.0
    assert bench._mean_tail([5.0]) == 5.0
