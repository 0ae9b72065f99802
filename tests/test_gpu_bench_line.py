"""bench.py end to end on the tiny workload (a child process): one JSON line
with the fields the benchmark promises, consistent with each other."""

import json
import os
import subprocess
import sys

import pytest

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(600)
def test_bench_json_line_tiny():
    print("[bench-line] tiny, 3 steps, graph replay", flush=True)
    r = subprocess.run([sys.executable, "bench.py", "--config", "tiny", "--steps", "3", "--warmup", "1", "--graph",
                        "--extra-configs", "gpt345m"],
                       cwd=ROOT, capture_output=True, text=True, timeout=540)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [x for x in r.stdout.splitlines() if x.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1 and d["dtype"] == "f32"
    assert d["config"]["workload"] == "tiny" and d["higher_is_better"] is True
    n = d["config"]["n_params"]
    assert d["value"] == pytest.approx(n / (d["ms_per_step"] * 1e-3), rel=1e-9)
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], rel=1e-9)
    assert rf["achieved"] == pytest.approx(rf["bytes_alg_per_step_pass"] / (rf["ms_per_step_pass"] * 1e-3) / 1e9,
                                           rel=1e-9)
    assert rf["launches_per_step_pass"] in (1, d["config"]["workers"])
    assert len(d["profiled_step_ms"]) == 3 and all(x > 0 for x in d["profiled_step_ms"])
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    assert cb["tiny_single_core"]["ms_per_step"] > 0
    assert d["graph"]["ms_per_step"] > 0
    assert d["bootstrap_step"]["ms"] > 0
    assert d["config"]["v_stored"] is False and d["step_storing_v"]["ms_per_step"] > 0
    sr = d["stream_reference"]
    assert sr["bytes"] == 12 * d["config"]["workers"] * n and sr["ms"] > 0
    assert sr["GBps"] == pytest.approx(sr["bytes"] / (sr["ms"] * 1e-3) / 1e9, rel=1e-9)
    ex = d["configs"]["gpt345m"]
    assert set(d["configs"]) == {"gpt345m"}
    assert ex["steps"] == 3 and ex["warmup"] == 1 and ex["workers"] == 8
    assert ex["params_per_s"] == pytest.approx(ex["n_params"] / (ex["ms_per_step"] * 1e-3), rel=1e-9)
    assert ex["hbm_frac_alg"] == pytest.approx(ex["hbm_gbps_alg"] / 8000.0, rel=1e-9)
    sp = ex["step_pass"]
    assert sp["frac"] == pytest.approx(sp["achieved"] / 8000.0, rel=1e-9)
    assert sp["achieved"] == pytest.approx(sp["bytes_alg_per_step_pass"] / (sp["ms_per_step_pass"] * 1e-3) / 1e9,
                                           rel=1e-9)
    assert 0 < sp["frac"] < 1 and len(ex["profiled_step_ms"]) == 3
    assert cb["cores"] <= cb["affinity_cores"]
