"""The benchmark's one-line JSON contract, on the GPU: the default run (the
headline prefill workload) and the decode workload each print exactly one
JSON line with the contracted keys, a roofline object and a CPU-oracle
baseline. Runs bench.py as a child process with a short step count."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KEYS = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
        "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"}


def run_bench(*args):
    print("case bench.py", " ".join(args), flush=True)
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                         timeout=240)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [l for l in res.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, res.stdout
    return json.loads(lines[0])


def check_line(b, steps, warmup):
    assert KEYS <= set(b), KEYS - set(b)
    assert b["n_gpus"] == 1 and b["steps"] == steps and b["warmup"] == warmup
    assert b["value"] > 0 and b["ms_per_step"] > 0 and b["higher_is_better"] is True
    assert b["ms_per_step_median"] > 0 and b["clock_settle"]["ms"] >= 50.0
    assert isinstance(b["config"], dict) and "workload" in b["config"]
    r = b["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert 0 < r["achieved"] < r["peak"] and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    c = b["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1 and c["sample"]


def test_bench_default_line():
    b = run_bench("--steps", "3", "--warmup", "1", "--cpu-seconds", "1", "--settle-ms", "50", "--cold-steps", "3")
    check_line(b, 3, 1)
    assert b["config"]["workload"].startswith("varlen8_h32") and b["dtype"] == "bf16"
    r = b["roofline"]
    assert 0 < r["frac_of_step"] < 1 and b["kernel_timing_pass"]["steps"] == 3
    assert b["mfma_roofline"]["flops_per_token_head"] == 118784
    h = b["host_per_call"]
    assert h["python_us"] > 0 and h["c_abi_us"] >= 0


def test_bench_decode_line():
    b = run_bench("--workload", "decode_n256_h32", "--steps", "3", "--warmup", "1", "--cpu-seconds", "1",
                  "--settle-ms", "50")
    check_line(b, 3, 1)
    assert b["config"]["workload"].startswith("decode_n256_h32")
