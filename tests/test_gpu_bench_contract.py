"""bench.py's output line on the single-matrix workload: one JSON object with
every field of the benchmark contract, consistent with itself."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_line_fields():
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--workload", "single",
                        "--steps", "2", "--warmup", "1"],
                       capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["unit"] == "GB/s" and d["higher_is_better"] is True and d["data"] == "synthetic"
    assert d["config"]["workload"] == "single"
    assert d["value"] > 0 and d["ms_per_step"] > 0
    # value is the input bytes over the timed steps' wall time
    assert abs(d["value"] - d["config"]["bf16_bytes"] / (d["ms_per_step"] / 1e3) / 1e9) <= 0.01 * d["value"] + 0.01
    rf = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in rf, k
    assert rf["peak"] == 8000.0 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    cb = d["cpu_baseline"]
    for k in ("value", "unit", "cores", "kind", "sample"):
        assert k in cb, k
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0
    # the timed steps' own outputs against the oracle on the baseline's sample
    pa = d["parity"]
    assert pa["entropy_max_rel_err"] < 1e-5
    assert pa["s_max_rel_err"] < 1e-4 and pa["t_max_rel_err"] < 1e-4
    assert pa["codes_mismatch_stage_isolated"] == 0 and pa["codes"] == 256 * 512

