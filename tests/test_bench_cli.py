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
    # three steps: one finalize per step, the reduce in one dispatch and the
    # update in two dispatches per step
    (out / f"prof_kt_{label}" / "x_kernel_stats.csv").write_text(
        '"Name","Calls","AverageNs","MinNs","MaxNs"\n'
        '"zk::(anonymous namespace)::k1_reduce_check(int)",3,2000,1900,2100\n'
        '"zk::(anonymous namespace)::k2_adam(int)",6,1500,1400,1600\n'
        '"zk::(anonymous namespace)::kf_reduce_finalize(int)",3,10,9,11\n'
        '"calib_copy(int)",2,1000,990,1010\n')
    for cname, calib_kib, k1, k2 in (("FETCH_SIZE", 2.0, 8.0, 4.0), ("WRITE_SIZE", 4.0, 4.0, 7.0)):
        d = out / f"prof_{cname}_{label}"
        d.mkdir()
        (out / f"bench_{cname}_{label}.log").write_text(json.dumps(line) + "\n")
        rows = ['"Kernel_Name","Counter_Name","Counter_Value"']
        rows += [f'"calib_copy(int)","{cname}",{calib_kib}']
        for _ in range(2):  # two steps in the counter runs
            rows += [f'"zk::(anonymous namespace)::k1_reduce_check(int)","{cname}",{k1}',
                     f'"zk::(anonymous namespace)::k2_adam(int)","{cname}",{k2}',
                     f'"zk::(anonymous namespace)::k2_adam(int)","{cname}",{k2}',
                     f'"zk::(anonymous namespace)::kf_reduce_finalize(int)","{cname}",0.5',
                     f'"other_kernel(int)","{cname}",99']
        (d / "y_counter_collection.csv").write_text("\n".join(rows) + "\n")
    bench.summarize_rocprof(label, "--workload demo", "--steps 1", out=str(out), prof=str(prof))
    rec = json.loads((prof / f"traffic_{label}.json").read_text())
    assert rec["fetch_scale"] == 4096 / (2.0 * 1024) and rec["write_scale"] == 4096 / (4.0 * 1024)
    k1, k2 = rec["kernels"]["k1_reduce_check"], rec["kernels"]["k2_adam"]
    assert k1["read_bytes"] == 8.0 * 1024 * 2.0 and k1["write_bytes"] == 4.0 * 1024 * 1.0
    assert k1["dispatches_per_step"] == 1 and k2["dispatches_per_step"] == 2
    # the update's two dispatches per step add up
    assert k2["read_bytes"] == 2 * 4.0 * 1024 * 2.0 and k2["write_bytes"] == 2 * 7.0 * 1024
    assert k1["algorithmic_bytes"] == (2 * N + 4) * S
    assert k2["algorithmic_bytes"] == 30 * S
    assert k2["bytes_per_step"] == k2["read_bytes"] + k2["write_bytes"]
    assert "other_kernel" not in rec["kernels"]
    md = (prof / f"k1_k2_{label}_hbm_traffic.md").read_text()
    assert "--summarize-rocprof demo" in md and "rocprofv3 --pmc FETCH_SIZE" in md
    stats = (prof / f"k1_k2_{label}_kernel_stats.md").read_text()
    # per step: 2 x 1.5 us of update dispatches, 30 S bytes over 3.0 us
    row = next(ln for ln in stats.splitlines() if ln.startswith("| k2_adam |"))
    cells = [c.strip() for c in row.strip("|").split("|")]
    assert cells[1] == "6" and cells[2] == "2" and cells[6] == "3.0"
    assert cells[8] == f"{30 * S / 3.0e3:.0f}"
