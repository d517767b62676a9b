"""bench.py's output contract, on the GPU: a short run of the tiny workload in
a child process prints one JSON line with the required keys, a roofline
entry for the dominant kernel and the CPU baseline of the oracle."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_the_contract_line(tmp_path):
    log_path = tmp_path / "steps.jsonl"
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--workload", "tiny", "--steps", "3",
                        "--warmup", "1", "--cpu-sample", str(1 << 16), "--log-steps", str(log_path)],
                       capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-4000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["scaling"] == "weak" and d["vs_baseline"] is None and d["data"] == "synthetic"
    assert d["config"]["workload"] == "tiny" and "model" not in d["config"]
    # whole-job throughput: parameters updated per second over the timed steps
    assert abs(d["value"] - d["config"]["params"] / (d["ms_per_step"] * 1e-3)) <= 1e-6 * d["value"]
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["achieved"] > 0 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-12
    assert rf["traffic"] is None or rf["traffic"] > 0
    mc = d["measured_ceilings"]
    assert mc["copy_gbps"] > 0 and mc["read_gbps"] > 0 and mc["runtime_copy_gbps"] > 0
    # per-step event times beside the wall-clock mean, on every stride-th step
    assert 0 < d["step_ms_min"] <= d["step_ms_median"]
    assert d["event_stride"] >= 1 and d["instrumented_steps"] == len(range(0, 3, d["event_stride"]))
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["unit"] == d["unit"]
    assert isinstance(cb["sample"], str) and cb["sample"]
    # timed on one thread and on the process's CPU share, both stated
    assert cb["one_thread"]["cores"] == 1 and cb["one_thread"]["value"] > 0
    assert cb["cores"] == cb["host"]["threads"] <= cb["host"]["affinity_cores"]
    # the per-step log: one line per extra step, after everything timed
    recs = [json.loads(ln) for ln in open(log_path)]
    assert len(recs) == 3
    assert [x["iter"] for x in recs] == [d["final_state"]["t"] + i for i in (1, 2, 3)]
    for x in recs:
        assert x["workload"] == "tiny" and x["found_inf"] == 0 and x["step_ms"] > 0 and x["call_ms"]
