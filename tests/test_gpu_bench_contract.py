"""bench.py end to end on the GPU, with a few steps: one JSON line whose
fields keep the benchmark's contract (the throughput of the whole step, a
roofline object for the partial kernel, the CPU oracle's timed baseline, the
parity of the timed outputs against that oracle run)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args, timeout=110):
    cmd = [sys.executable, os.path.join(ROOT, "bench.py")] + list(args)
    print("bench:", " ".join(args), flush=True)
    return subprocess.run(cmd, capture_output=True, text=True, timeout=timeout, cwd=ROOT)


def test_bench_prints_one_json_line_with_the_contract_fields():
    r = run_bench("--steps", "8", "--warmup", "2", "--also", "llama8b_b16_ragged_f16",
                  "--also-steps", "8", "--cpu-budget", "0.5", "--cold-calls", "4")
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 8 and d["warmup"] == 2
    assert d["unit"] == "GB/s" and d["higher_is_better"] is True and d["data"] == "synthetic"
    assert d["vs_baseline"] is None
    assert d["config"]["workload"] == "llama1b_ctx3060_f16"
    # Whole-step throughput: the step's K/V bytes over the measured step time.
    kv = d["config"]["kv_bytes_per_step"]
    assert kv == 2 * 3060 * 8 * 64 * 2
    assert d["value"] == pytest.approx(kv / (d["ms_per_step"] * 1e-3) / 1e9, rel=2e-3)
    assert 0 < d["value"] < 8000
    rl = d["roofline"]
    assert rl["bound"] == "hbm" and rl["unit"] == "GB/s" and rl["peak"] == 8000
    assert 0 < rl["frac"] <= 1 and rl["frac"] == pytest.approx(rl["achieved"] / rl["peak"], rel=1e-3)
    # The partial kernel's event time (eager launches) stays near the graph
    # step it is part of.
    assert 0 < rl["kernel_us"] < d["ms_per_step"] * 1e3 * 1.5
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["cores"] >= 1 and cpu["value"] > 0 and cpu["sample"]
    par = d["parity"]
    assert par["out_rel_l2"] <= 1e-3 and par["row_excess_max"] <= 1e-3, par
    assert par["lse_max_abs_err"] <= 1e-4, par
    assert "llama8b_b16_ragged_f16" in d["also"]
    a = d["also"]["llama8b_b16_ragged_f16"]
    assert a["us_per_step"] > 0 and 0 < a["partial_frac"] <= 1
