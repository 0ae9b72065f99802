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
    # as K passes: every pass reads the mask words, and the K - 1 non-owner
    # sparse buffers are written and read back
    for v_out in (False, True):
        multi = bench.alg_bytes_step_pass(n, P, K, k, v_out, passes=K)
        assert multi - bench.alg_bytes_step_pass(n, P, K, k, v_out) == (K - 1) * n / 8 + 8 * (K - 1) * P * k
        assert multi < bench.alg_bytes_step(n, P, K, k, v_out)


def _write_csv(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


OWNER = ("void scape::(anonymous namespace)::compress_kernel<true, true, true, false, 2>(scape::Geom, float const*, "
         "float*, unsigned long const*, unsigned int const*, float*, float*, float*, float*, float*, "
         "scape::(anonymous namespace)::AdamsC, unsigned int const*, unsigned long*, unsigned int*, unsigned int*, "
         "int, long, float const*, int)")
OWNER_V = OWNER.replace("<true, true, true, false, 2>", "<true, true, true, true, 2>")
WORKER = OWNER.replace("<true, true, true, false, 2>", "<false, true, false, false, 1>")
COMP = OWNER.replace("<true, true, true, false, 2>", "<false, true, false, false, 0>")
HDR_S = ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"]


def test_prof_summary_short_names_and_roles():
    from sparse_communication_distributed_amd.prof_summary import short_name, step_pass_role
    assert short_name(OWNER) == "compress_kernel<true, true, true, false, 2>"
    assert short_name("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"
    assert short_name("void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float>, "
                      "std::array<char*, 1ul> >(int, at::native::FillFunctor<float>, std::array<char*, 1ul>)") \
        == "vectorized_elementwise_kernel<…>"
    assert short_name("void scape::(anonymous namespace)::zero_u32_kernel(unsigned int*, long)") == "zero_u32_kernel"
    assert [step_pass_role(x) for x in (OWNER, OWNER_V, WORKER, COMP)] == ["owner", "owner_v", "worker", None]
    small = OWNER.replace("<true, true, true, false, 2>", "<true, true, true, false, 3>")
    assert step_pass_role(small) == "owner"  # the latency form of the single pass


def test_prof_summary_step_pass_of_k_launches(tmp_path):
    """K = 4: three worker passes and one owner pass per step.  The step
    pass time and traffic are the owner pass's plus three worker passes'."""
    stats = tmp_path / "stats.csv"
    # 3 v-less steps and 2 v-storing steps: 15 worker launches
    _write_csv(stats, HDR_S, [[OWNER, 3, 30e6, 10e6, 50.0, 9e6, 11e6, 1.0],
                              [WORKER, 15, 60e6, 4e6, 40.0, 3.9e6, 4.1e6, 1.0],
                              [OWNER_V, 2, 22e6, 11e6, 5.0, 11e6, 11e6, 0.0],
                              [COMP, 1, 5e6, 5e6, 5.0, 5e6, 5e6, 0.0]])
    stats2 = tmp_path / "stats2.csv"  # a second profiled process, slower placement
    _write_csv(stats2, HDR_S, [[WORKER, 15, 75e6, 5e6, 40.0, 4.9e6, 5.1e6, 1.0],
                               [OWNER, 3, 36e6, 12e6, 50.0, 11e6, 13e6, 1.0],
                               [OWNER_V, 2, 26e6, 13e6, 10.0, 13e6, 13e6, 0.0]])
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    # two steps: the first step's launches (1 owner, 3 workers) are dropped;
    # the calibration copy reads 1 GiB but its FETCH_SIZE counter shows half of it
    f_rows = [["__amd_rocclr_copyBuffer", "FETCH_SIZE", 524288]]
    w_rows = [["__amd_rocclr_copyBuffer", "WRITE_SIZE", 1048576]]
    for step in range(2):
        for _ in range(3):
            f_rows.append([WORKER, "FETCH_SIZE", 9 if step == 0 else 300])
            w_rows.append([WORKER, "WRITE_SIZE", 9 if step == 0 else 100])
        f_rows.append([OWNER, "FETCH_SIZE", 9 if step == 0 else 1000])
        w_rows.append([OWNER, "WRITE_SIZE", 9 if step == 0 else 500])
    f_rows.append([COMP, "FETCH_SIZE", 7000])
    _write_csv(fetch, hdr, f_rows)
    _write_csv(write, hdr, w_rows)
    out = tmp_path / "prof"
    r = subprocess.run([sys.executable, "-m", "sparse_communication_distributed_amd.prof_summary", "--stats", str(stats),
                        "--stats", str(stats2),
                        "--fetch", str(fetch), "--write", str(write), "--workload", "x", "--out", str(out)],
                       cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    doc = json.load(open(str(out) + "_counters.json"))
    assert doc["kernels"] == {"owner": "compress_kernel<true, true, true, false, 2>",
                              "worker": "compress_kernel<false, true, false, false, 1>"}
    assert doc["worker_passes_per_step"] == pytest.approx(3.0)
    assert doc["fetch_scale"] == pytest.approx(2.0)
    assert doc["write_scale"] == pytest.approx(1.0)
    # KiB -> bytes, scaled: owner + 3 workers
    assert doc["hbm_read_bytes_per_step_pass"] == pytest.approx((1000 + 3 * 300) * 1024 * 2.0)
    assert doc["hbm_write_bytes_per_step_pass"] == pytest.approx((500 + 3 * 100) * 1024)
    # per process: owner average + 15 / 5 worker averages
    assert doc["step_pass_ms_per_process"] == pytest.approx([10.0 + 3 * 4.0, 12.0 + 3 * 5.0])
    md = open(str(out) + ".md").read()
    assert "| 2 | 12.000 | 5.000 | 3.00 | 27.000 |" in md and "worker passes, then the owner pass" in md
    assert "| compress_kernel<true, true, true, true, 2> | 2 |" in md


def test_step_pass_hash_ignores_comments_only():
    """The counters file stays valid across comment and layout edits of the
    step pass's sources, and not across code edits."""
    from sparse_communication_distributed_amd.prof_summary import _code_only
    a = "int f(int x) {  // doubles\n  return 2 * x; /* no\n overflow */ }\n"
    b = "int f(int x) {\n    return 2 * x;\n}\n"
    c = "int f(int x) { return 3 * x; }"
    assert _code_only(a) == _code_only(b)
    assert _code_only(a) != _code_only(c)


def test_extra_workloads_selection():
    sys.path.insert(0, ROOT)
    import bench
    names = ["tiny", "gpt345m", "llama500m", "llama1.8b", "stress"]
    assert bench.extra_workloads("all", "llama1.8b", names) == ["tiny", "gpt345m", "llama500m", "stress"]
    assert bench.extra_workloads("none", "llama1.8b", names) == []
    assert bench.extra_workloads("stress, tiny", "llama1.8b", names) == ["tiny", "stress"]
    assert bench.extra_workloads("tiny", "tiny", names) == []
    with pytest.raises(SystemExit):
        bench.extra_workloads("gpt2", "tiny", names)


def test_counter_calibration_ignores_small_copies():
    """The calibration uses the 1 GiB copies only, not the workload's own
    copies through the same copy kernel: small uploads and read-backs, and
    whole error-feedback buffers moved while their placement is chosen."""
    from sparse_communication_distributed_amd.prof_summary import calibration_values
    gib = [524288.0, 524280.0, 524300.0]   # FETCH_SIZE reads half of a 1 GiB copy
    small = [3.0, 12.5, 0.0, 400.0]
    placement = [14.2e6, 14.2e6, 28.4e6]   # 28 GB buffers moved between allocations
    assert sorted(calibration_values(gib + small + placement)) == sorted(gib)
    assert sorted(calibration_values([1048576.0, 1048570.0] + placement)) == [1048570.0, 1048576.0]
    with pytest.raises(SystemExit, match="calibration"):
        calibration_values(small + placement)
