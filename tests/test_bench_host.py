"""bench.py's host logic, on the CPU: the stream-mix probes move exactly the
bytes the byte model gives each kernel, the counter summary derives its
ratios from the right counters, and the CPU share follows the affinity
mask, the cgroup quota and OMP_NUM_THREADS."""
import csv
import os

import pytest

import bench
from synth import workloads

NAMES = ("tiny", "gpt2_small", "zero3_rank_7b", "unsharded_7b", "tp_column_slice")


@pytest.mark.parametrize("name", NAMES)
@pytest.mark.parametrize("single", [False, True])
def test_mix_bytes_equal_the_byte_model(name, single):
    """Per element and replica, a kind's mix reads and writes what the byte
    model charges one launch of that kind per parameter (the read-modify-
    write launch covers every replica, the mix one)."""
    w = workloads.by_name(name)
    if single and w.max_norm > 0:
        pytest.skip("the single pass needs a workload without clipping")
    per = bench.bytes_model(w, single)
    for kind, b in per.items():
        spec = bench.mix_spec(w, kind)
        if spec is None:
            assert kind == "accumulate_first"
            continue
        mix_bytes = 2 * spec["r16"] + 4 * spec["r32"] + 4 * spec["w32"] + 2 * spec["w16"]
        launches = {"accumulate": max(1, (1 if w.partials else w.a) - 2)}.get(kind, 1)
        per_launch = b / launches
        if kind == "accumulate":
            assert per_launch == w.n * mix_bytes
        else:
            assert per_launch == mix_bytes, (name, kind, per_launch, spec)


def test_counter_summary_ratios(tmp_path):
    path = tmp_path / "run_counter_collection.csv"
    rows = []
    for disp, (name, vals) in enumerate([
        ("void dpk::k_reduce_adamw<1, 2, 8, 2>(...)", {"TCC_EA0_RDREQ_sum": 100.0, "TCC_EA0_RDREQ_LEVEL_sum": 25000.0,
                                                      "TCC_EA0_WRREQ_sum": 50.0, "TCC_EA0_WRREQ_LEVEL_sum": 5000.0,
                                                      "TCC_CYCLE_sum": 1000.0,
                                                      "TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum": 40.0}),
        ("stream_read(...)", {"TCC_EA0_RDREQ_sum": 10.0, "TCC_EA0_RDREQ_LEVEL_sum": 3000.0})]):
        for c, v in vals.items():
            rows.append({"Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": c, "Counter_Value": v,
                         "Start_Timestamp": 1000, "End_Timestamp": 3000})
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=list(rows[0]))
        wr.writeheader()
        wr.writerows(rows)
    out = bench.summarize_pmc([str(path)])
    assert "### reduce_adamw: 1 dispatches, 2.0 us" in out
    assert "| *read latency (L2 cycles per request)* | 250 |" in out
    assert "| *write latency (L2 cycles per request)* | 100 |" in out
    assert "| *read DRAM-credit stall share of L2 cycles* | 0.04 |" in out
    assert "### read_probe" in out and "| *read latency (L2 cycles per request)* | 300 |" in out


def test_cpu_share(tmp_path, monkeypatch):
    monkeypatch.setattr(os, "sched_getaffinity", lambda pid: set(range(64)))
    monkeypatch.delenv("OMP_NUM_THREADS", raising=False)
    missing = str(tmp_path / "none")
    assert bench.cpu_share(missing)["threads"] == 64
    cpu_max = tmp_path / "cpu.max"
    cpu_max.write_text("1600000 100000\n")
    share = bench.cpu_share(str(cpu_max))
    assert share == {"affinity_cores": 64, "cgroup_quota_cores": 16, "omp_num_threads": None, "threads": 16}
    cpu_max.write_text("max 100000\n")
    assert bench.cpu_share(str(cpu_max))["threads"] == 64
    monkeypatch.setenv("OMP_NUM_THREADS", "8")
    assert bench.cpu_share(str(cpu_max))["threads"] == 8


def test_event_stride():
    # timing events cost at most about 2% of the timed region: a step of a
    # few milliseconds carries them on every step, a 40 us step on few
    assert bench.event_stride(None, 3) == 1
    assert bench.event_stride(0.1, 9) == 1
    assert bench.event_stride(1e-3, 11) == 3
    assert bench.event_stride(2.5e-3, 11) == 1
    s = bench.event_stride(40e-6, 3)
    assert s == 15 and 3 * bench.EVENT_RECORD_US * 1e-6 / (s * 40e-6) <= bench.EVENT_BUDGET
