"""The benchmark's output line on the GPU: one JSON object with the fields the
harness reads, the roofline of the decode kernels, the read ceiling and the
oracle timed on the host (a short run: 8 steps over 2 layer pools)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_complete_json_line():
    print("bench.py --steps 8 --warmup 2 --layers 2 --cpu-reps 1", flush=True)
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "8",
                          "--warmup", "2", "--layers", "2", "--cpu-reps", "1"],
                         capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [ln for ln in res.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, res.stdout[-2000:]
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 8 and d["warmup"] == 2
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["unit"] == "GB/s"
    assert d["dtype"] == "bf16" and "workload" in d["config"]
    roof = d["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert 0 < roof["frac"] < 1
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert "traffic" in roof
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["sample"]
    rc = d["read_ceiling"]
    assert rc["kernel"] == "pa_read_tiles" and rc["us"] > 0
    # the loads alone cannot take longer than the decode that makes them (a
    # single short phase can catch a slow moment of the machine: the median
    # over graph replays is the steadier figure)
    assert rc["us"] <= max(d["decode_us"], d["decode_us_spread"]["median"]) * 1.1
    # the plain entry point is reported beside the host-planned partition
    # length; its automatic split plans the length on the device here
    assert d["config"]["partition_plan"] == "pa_decode_plan (host context lengths)"
    plain = d["decode_plain"]
    assert plain["entry"].startswith("pa_decode (automatic partitions: length planned on "
                                     "the device") and plain["us"] > 0
    assert abs(plain["frac_of_peak"] * 8000.0 - plain["GBps"]) < 1.0
