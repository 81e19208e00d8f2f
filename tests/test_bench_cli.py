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
