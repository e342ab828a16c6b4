"""bench.py's command line on the host: the one-GPU rule and the oracle-only
timing mode (no GPU needed for either)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_cpu_only_times_every_real_row_of_the_small_workload():
    r = run("--config", "tiny", "--cpu-only", "--cpu-budget", "0")
    assert r.returncode == 0, r.stderr
    line = json.loads(r.stdout.strip().splitlines()[-1])
    cb = line["cpu_baseline"]
    assert line["config"]["workload"] == "tiny"
    assert cb["kind"] == "oracle" and cb["unit"] == "TFLOP/s" and cb["value"] > 0
    # tiny has 128 real rows; budget 0 walks all of them
    assert "on 128 random real rows" in cb["sample"]
