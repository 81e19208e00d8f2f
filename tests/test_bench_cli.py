"""bench.py's command-line contract on the CPU: one GPU only, the
single-pass mode refuses workloads that clip, and the CPU oracle baseline
reports its one-process and all-processes figures."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, cwd=ROOT, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_one_pass_refuses_a_clipped_workload():
    r = _run("--workload", "llama3_8b", "--one-pass", "--no-cpu-baseline")
    assert r.returncode == 2
    assert "without clipping" in r.stderr


def test_bytes_per_param():
    sys.path.insert(0, ROOT)
    import bench
    assert bench.bytes_per_param(8) == (20, 30)
    assert bench.bytes_per_param(64) == (132, 30)


def test_cpu_baseline_reports_both_figures():
    sys.path.insert(0, ROOT)
    import bench
    import synth
    r = bench.cpu_baseline(synth.TINY, 0.2, 2)
    assert r["kind"] == "oracle" and r["unit"] == "params/s"
    assert r["cores"] == 2 and r["value"] > 0
    assert r["single_process"]["cores"] == 1 and r["single_process"]["value"] > 0
    one = bench.cpu_baseline(synth.TINY, 0.2, 1)
    assert one["cores"] == 1 and one["value"] == one["single_process"]["value"]


if __name__ == "__main__":
    sys.exit(pytest.main([__file__, "-q"]))


def test_summarize_rocprof_scales_by_the_calibration_copy(tmp_path):
    """--summarize-rocprof on made-up rocprofv3 output: the counter scale is
    the calibration copy's known bytes over what the counter read for it, and
    each kernel's bytes are compared with its algorithmic bytes."""
    import json
    sys.path.insert(0, ROOT)
    import bench

    out, prof = tmp_path / "out", tmp_path / "prof"
    prof.mkdir()
    label, S, N = "demo", 1000, 8
    line = {"metric": "params updated/sec + achieved HBM GB/s, demo shard step",
            "config": {"shard": S, "world_size_simulated": N, "workload": "demo workload"},
            "kernels": {"k1_reduce_check": {"ms": 1.0, "gbps": 20.0}},
            "ms_per_step": 2.0, "value": 5e5, "calibration_copy": {"bytes": 4096}}
    (out / f"prof_kt_{label}").mkdir(parents=True)
    (out / f"bench_kt_{label}.log").write_text("noise\n" + json.dumps(line) + "\n")
    (out / f"prof_kt_{label}" / "x_kernel_stats.csv").write_text(
        '"Name","Calls","AverageNs","MinNs","MaxNs"\n'
        '"zk::(anonymous namespace)::k1_reduce_check(int)",3,2000,1900,2100\n'
        '"zk::(anonymous namespace)::k2_adam(int)",3,3000,2900,3100\n'
        '"calib_copy(int)",2,1000,990,1010\n')
    for cname, calib_kib, k1, k2 in (("FETCH_SIZE", 2.0, 8.0, 8.0), ("WRITE_SIZE", 4.0, 4.0, 14.0)):
        d = out / f"prof_{cname}_{label}"
        d.mkdir()
        (out / f"bench_{cname}_{label}.log").write_text(json.dumps(line) + "\n")
        rows = ['"Kernel_Name","Counter_Name","Counter_Value"']
        rows += [f'"calib_copy(int)","{cname}",{calib_kib}',
                 f'"zk::(anonymous namespace)::k1_reduce_check(int)","{cname}",{k1}',
                 f'"zk::(anonymous namespace)::k2_adam(int)","{cname}",{k2}',
                 f'"other_kernel(int)","{cname}",99']
        (d / "y_counter_collection.csv").write_text("\n".join(rows) + "\n")
    bench.summarize_rocprof(label, "--workload demo", "--steps 1", out=str(out), prof=str(prof))
    rec = json.loads((prof / f"traffic_{label}.json").read_text())
    assert rec["fetch_scale"] == 4096 / (2.0 * 1024) and rec["write_scale"] == 4096 / (4.0 * 1024)
    k1 = rec["kernels"]["k1_reduce_check"]
    assert k1["read_bytes"] == 8.0 * 1024 * 2.0 and k1["write_bytes"] == 4.0 * 1024 * 1.0
    assert k1["algorithmic_bytes"] == (2 * N + 4) * S
    assert rec["kernels"]["k2_adam"]["algorithmic_bytes"] == 30 * S
    assert "other_kernel" not in rec["kernels"]
    md = (prof / f"k1_k2_{label}_hbm_traffic.md").read_text()
    assert "--summarize-rocprof demo" in md and "rocprofv3 --pmc FETCH_SIZE" in md
    assert (prof / f"k1_k2_{label}_kernel_stats.md").exists()
