"""The JSON line bench.py prints (GPU): one line, the fields and units the
measurement contract names, a roofline fraction that is achieved over peak, and
one suite entry per other workload.  Short runs (two timed steps, no counter
passes, no CPU baseline) in a child process.
"""
import json
import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
METRIC = "varlen paged attention: prefill TFLOP/s (%MFMA peak); decode KV GB/s (%HBM)"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bench(args):
    print("bench.py", " ".join(args), flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, cwd=ROOT,
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.strip().splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


def _check_roofline(rl):
    assert rl["bound"] in ("hbm", "mfma")
    assert rl["unit"] == ("GB/s" if rl["bound"] == "hbm" else "TFLOP/s")
    assert rl["peak"] == (8000.0 if rl["bound"] == "hbm" else 2500.0)
    assert rl["achieved"] > 0 and abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-3
    assert rl["traffic"] is None or rl["traffic"] > 0


def test_headline_line():
    d = _bench(["--gpus", "1", "--steps", "2", "--warmup", "1", "--no-counters", "--no-cpu-baseline"])
    assert d["metric"] == METRIC
    assert d["unit"] == "TFLOP/s" and d["value"] > 0 and d["higher_is_better"] is True
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1 and d["ms_per_step"] > 0
    assert d["dtype"] == "bf16" and d["vs_baseline"] is None and isinstance(d["data"], str)
    assert d["config"]["workload"].startswith("c4")
    # value is the step's algorithmic flops over its time
    assert abs(d["value"] - d["detail"]["tflops_per_step"]) < 1e-2
    _check_roofline(d["roofline"])
    assert d["roofline"]["bound"] == "mfma"
    assert sorted(d["suite"]) == ["c1", "c2", "c3", "c5a", "c5b"]
    for name, e in d["suite"].items():
        assert e["value"] > 0 and e["ms_per_step"] > 0, name
        assert e["unit"] == ("GB/s" if name in ("c2", "c5a", "c5b") else "TFLOP/s"), name


def test_single_decode_workload_line():
    d = _bench(["--workload", "c2", "--steps", "2", "--warmup", "1", "--no-cpu-baseline"])
    assert d["metric"] == METRIC and d["unit"] == "GB/s" and d["value"] > 0
    assert d["config"]["workload"].startswith("c2")
    _check_roofline(d["roofline"])
    assert d["roofline"]["bound"] == "hbm"
