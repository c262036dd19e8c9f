"""The bench line's contract, on the tiny workload: one JSON line with the
metric fields, a roofline object whose fraction is achieved / peak, and a
CPU-oracle baseline object that names its sample and core count."""

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    print(f"[case] bench.py {' '.join(args)}", flush=True)
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                         capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [l for l in res.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, res.stdout
    return json.loads(lines[0])


def test_bench_line_contract_tiny():
    d = _bench("--workload", "tiny", "--steps", "3", "--warmup", "1", "--cpu-budget", "2")
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["vs_baseline"] is None
    assert "workload" in d["config"]
    roof = d["roofline"]
    assert roof["bound"] in ("hbm", "mfma")
    assert roof["unit"] == ("GB/s" if roof["bound"] == "hbm" else "TFLOP/s")
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    if d.get("clock"):                        # SMU reading of a sustained loop of the step
        assert 0 < d["clock"]["gfxclk_mhz"] < 5000 and d["clock"]["socket_power_w"] > 0
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["sample"]
