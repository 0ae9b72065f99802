"""bench.py's command line and the profile summarizer, on the CPU."""

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_bytes_formula():
    sys.path.insert(0, ROOT)
    import bench
    # Llama-1.8B layout, 99% sparsity: 94.42 GB per step, 94.49 GB storing v
    n, P, K, k = 1_775_372_288, 32, 4, 554_803
    assert abs(bench.alg_bytes_step(n, P, K, k) / 1e9 - 94.423) < 0.01
    assert abs(bench.alg_bytes_step(n, P, K, k, True) / 1e9 - 94.494) < 0.01
    assert bench.alg_bytes_step(n, P, K, k, True) - bench.alg_bytes_step(n, P, K, k) == 4 * P * k
    # the step pass moves everything except the emitted index list and the read-back of b
    for v_out in (False, True):
        assert bench.alg_bytes_step_pass(n, P, K, k, v_out) < bench.alg_bytes_step(n, P, K, k, v_out)
    assert bench.alg_bytes_step_pass(n, P, K, k, True) - bench.alg_bytes_step_pass(n, P, K, k) == 4 * P * k


def _write_csv(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


STEP = ("void scape::(anonymous namespace)::compress_kernel<true, true, true, false>(scape::Geom, float const*, "
        "float*, unsigned long const*, unsigned int const*, float*, float*, float*, float*, float*, "
        "scape::(anonymous namespace)::AdamsC, unsigned int const*, unsigned long*, unsigned int*, unsigned int*, "
        "int, long, float const*)")
STEP_V = STEP.replace("<true, true, true, false>", "<true, true, true, true>")
COMP = STEP.replace("<true, true, true, false>", "<false, true, false, false>")


def test_prof_summary_short_names():
    from sparse_communication_distributed_amd.prof_summary import is_step_pass, short_name
    assert short_name(STEP) == "compress_kernel<true, true, true, false>"
    assert short_name("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"
    assert short_name("void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float>, "
                      "std::array<char*, 1ul> >(int, at::native::FillFunctor<float>, std::array<char*, 1ul>)") \
        == "vectorized_elementwise_kernel<…>"
    assert short_name("void scape::(anonymous namespace)::zero_u32_kernel(unsigned int*, long)") == "zero_u32_kernel"
    assert is_step_pass(STEP) and not is_step_pass(STEP_V) and not is_step_pass(COMP)


def test_prof_summary_scales_counters_by_the_copy(tmp_path):
    hdr_s = ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"]
    stats = tmp_path / "stats.csv"
    _write_csv(stats, hdr_s, [[STEP, 3, 60e6, 20e6, 80.0, 19e6, 21e6, 1.0],
                              [STEP_V, 2, 50e6, 25e6, 10.0, 24e6, 26e6, 1.0],
                              [COMP, 1, 5e6, 5e6, 10.0, 5e6, 5e6, 0.0]])
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    # the calibration copy reads 1 GiB but its FETCH_SIZE counter shows half of it;
    # the v-storing and component launches are not the step pass
    _write_csv(fetch, hdr, [["__amd_rocclr_copyBuffer", "FETCH_SIZE", 524288],
                            [STEP, "FETCH_SIZE", 999], [STEP_V, "FETCH_SIZE", 5000], [STEP, "FETCH_SIZE", 1000],
                            [COMP, "FETCH_SIZE", 7000], [STEP, "FETCH_SIZE", 1000]])
    _write_csv(write, hdr, [["__amd_rocclr_copyBuffer", "WRITE_SIZE", 1048576],
                            [STEP, "WRITE_SIZE", 7], [STEP, "WRITE_SIZE", 500], [STEP_V, "WRITE_SIZE", 9000],
                            [STEP, "WRITE_SIZE", 500]])
    stats2 = tmp_path / "stats2.csv"  # a second profiled process, slower placement
    _write_csv(stats2, hdr_s, [[STEP_V, 2, 50e6, 25e6, 10.0, 24e6, 26e6, 1.0],
                               [STEP, 3, 66e6, 22e6, 90.0, 21e6, 23e6, 1.0]])
    out = tmp_path / "prof"
    r = subprocess.run([sys.executable, "-m", "sparse_communication_distributed_amd.prof_summary", "--stats", str(stats),
                        "--stats", str(stats2),
                        "--fetch", str(fetch), "--write", str(write), "--workload", "x", "--out", str(out)],
                       cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    doc = json.load(open(str(out) + "_counters.json"))
    assert doc["kernel"] == "compress_kernel<true, true, true, false>"
    assert doc["fetch_scale"] == pytest.approx(2.0)
    assert doc["write_scale"] == pytest.approx(1.0)
    # first launch skipped; KiB -> bytes, scaled
    assert doc["hbm_read_bytes_per_launch"] == pytest.approx(1000 * 1024 * 2.0)
    assert doc["hbm_write_bytes_per_launch"] == pytest.approx(500 * 1024)
    assert doc["step_pass_avg_ms_per_process"] == pytest.approx([20.0, 22.0])
    md = open(str(out) + ".md").read()
    assert "compress_kernel (step pass, no v stored) in each profiled process" in md and "| 2 | 22.000 |" in md
    assert "| compress_kernel<true, true, true, true> | 2 |" in md


def test_step_pass_hash_ignores_comments_only():
    """The counters file stays valid across comment and layout edits of the
    step pass's sources, and not across code edits."""
    from sparse_communication_distributed_amd.prof_summary import _code_only
    a = "int f(int x) {  // doubles\n  return 2 * x; /* no\n overflow */ }\n"
    b = "int f(int x) {\n    return 2 * x;\n}\n"
    c = "int f(int x) { return 3 * x; }"
    assert _code_only(a) == _code_only(b)
    assert _code_only(a) != _code_only(c)
