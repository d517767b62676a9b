"""Benchmark of the data-parallel gradient reduce + AdamW step on one MI355X.

One step is the whole path over one batch of synthetic input that is already
resident in HBM: n*a micro-step accumulations (or none, for incoming
partials), the replica reduction with fused statistics, the finalisation of
the per-step scalars and the fused AdamW update of every parameter.

Prints one JSON line: params updated per second (``value``), the achieved HBM
bandwidth of the whole step under the algorithmic byte model, a roofline entry
for the dominant kernel (per-launch durations from HIP events recorded on the
stream the kernels run on) and the CPU oracle timed on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time
from typing import Optional

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X published HBM3E bandwidth
RESIDENT_GRAD_BUDGET = 80e9  # bytes of pre-generated gradients kept in HBM
CPU_BASELINE_SECONDS = 10.0  # oracle work timed for each leg of the CPU baseline
EVENT_RECORD_US = 4.0  # host time of one timing-event record on the step's stream (ROCm 7, MI355X host)
EVENT_BUDGET = 0.02  # the share of the timed region the timing events may cost
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SRC = (os.path.join(ROOT, "gradient_reduce_adam_amd", "csrc", "kernels.hip"),
              os.path.join(ROOT, "gradient_reduce_adam_amd", "csrc", "dp_internal.h"))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="unsharded_7b",
                    help="tiny | gpt2_small | zero3_rank_7b | unsharded_7b | tp_column_slice")
    ap.add_argument("--cpu-sample", type=int, default=1 << 26, help="params in the oracle's timed sample")
    ap.add_argument("--zero3-placements", type=int, default=3, metavar="K",
                    help="with the default workload: also time the ZeRO-3 rank share's single pass in this process "
                         "at K HBM placements (its state allocated behind spacers of 0, 3, 6, ... GiB) and report "
                         "the median and the range as an extra key; 0 to skip")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--chunk", type=int, default=0, help="chunk_elems of the plan (0: library default)")
    ap.add_argument("--bind", choices=("flat", "tensors", "grads"), default="flat",
                    help="bind every role as a flat buffer; every role through per-tensor pointer tables (same "
                         "memory), the gradients rebound before every micro-step (tensors); or only the gradients "
                         "per tensor, as a framework with per-tensor gradient buffers and the library's flat state "
                         "would (grads)")
    ap.add_argument("--update", choices=("auto", "two-pass", "single-pass"), default="auto",
                    help="two-pass: reduce, statistics, then the update; single-pass: reduce, statistics and the "
                         "update in one read of the state (runs without clipping); auto: single-pass when the "
                         "workload does not clip")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of one step captured into a HIP graph (the per-kernel times still come from "
                         "an eager timed run)")
    ap.add_argument("--layout", choices=("auto", "packed", "spread"), default="auto",
                    help="HBM placement of the update's arrays (see driver.DPStep)")
    ap.add_argument("--state", choices=("hbm", "host"), default="hbm",
                    help="where master, m and v live: HBM, or pinned host memory that the update kernels read and "
                         "write across PCIe (the offload variant)")
    ap.add_argument("--offload", choices=("direct", "staged"), default="direct",
                    help="with --state host: the kernels access the host state directly, or it is copied through "
                         "device slots on two copy streams (two-pass update only)")
    ap.add_argument("--checkpoint-dir", default="", metavar="DIR",
                    help="after the timed steps, save the state to DIR as 8 shards and restore it as 4, and print "
                         "a second JSON line with the save and restore rates")
    ap.add_argument("--overlap", default="", metavar="MB,MB,...",
                    help="instead of the step benchmark: a synthetic backward pass (matrix-core compute of "
                         "4 flops per parameter and token, then the gradients) with the last micro-step's "
                         "reduction in buckets of these sizes, sequential and overlapped on a second stream; "
                         "one JSON line per bucket size")
    ap.add_argument("--micro-buckets", action="store_true",
                    help="with --overlap: the earlier micro-steps are also accumulated bucket by bucket as the "
                         "backward pass produces them (dp_accumulate_all_range), overlapped in the same way")
    ap.add_argument("--tokens", type=int, default=4096, help="tokens per micro-batch of the synthetic backward")
    ap.add_argument("--log-steps", default="", metavar="FILE",
                    help="after everything timed, run --steps more steps, each followed by a read of the scalar "
                         "state (a synchronisation), and write one JSON line per step to FILE: t, iter, found_inf, "
                         "the loss scale, the norm, the clip factor and the time of each call")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="first run a plain device copy of BYTES bytes (3 times), as the reference kernel of the "
                         "FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="CSV",
                    help="print a table of the per-dispatch averages of every counter in these rocprofv3 --pmc "
                         "counter_collection.csv files, per kernel kind, with the derived latencies and stall "
                         "shares, then exit")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, then WRITE_SIZE) of a "
                         "--copy-calibration run into profiles/traffic.json, then exit")
    args = ap.parse_args()
    if args.steps < 1 or args.warmup < 0:
        ap.error("need --steps >= 1 and --warmup >= 0")
    return args


# rocprofv3 kernel names of each call kind (regular expressions on the
# demangled name; template arguments: addressing, dtype, first micro-step)
KERNEL_NAMES = {
    "accumulate_first": r"k_accumulate_all<\w+, \d, true>",
    "accumulate": r"k_accumulate_all<\w+, \d, false>",
    "accumulate_reduce": r"k_reduce<",
    "adamw": r"k_adamw<",
    "reduce_adamw": r"k_reduce_adamw<",
}
COPY_KERNEL = "copyBuffer"  # the runtime's plain device-to-device copy


def summarize_counters(fetch_csv: str, write_csv: str, workload: str, calib_bytes: int) -> dict:
    """Per-launch HBM bytes of each kernel kind from the FETCH_SIZE and
    WRITE_SIZE counters (KiB per dispatch), each scaled by the factor that
    maps the same counter on a plain copy of calib_bytes to the bytes that
    copy must move (calib_bytes read, calib_bytes written)."""
    import csv

    def load(path, counter):
        rows, first_copy = {}, None
        for r in sorted(csv.DictReader(open(path)), key=lambda r: int(r["Dispatch_Id"])):
            if r.get("Counter_Name", counter) != counter:
                continue
            name = r.get("Kernel_Name", "")
            rows.setdefault(name, []).append(float(r["Counter_Value"]))
            if first_copy is None and COPY_KERNEL in name:
                first_copy = float(r["Counter_Value"])  # the calibration copies run first
        return rows, first_copy

    fetch, f_kib = load(fetch_csv, "FETCH_SIZE")
    write, w_kib = load(write_csv, "WRITE_SIZE")

    import re

    def per_kind(rows, key):
        vals = [v for name, vs in rows.items() if re.search(key, name) for v in vs]
        return sum(vals) / len(vals) if vals else None

    f_fac = calib_bytes / (f_kib * 1024.0)
    w_fac = calib_bytes / (w_kib * 1024.0)
    out = {}
    for kind, key in KERNEL_NAMES.items():
        fk, wk = per_kind(fetch, key), per_kind(write, key)
        if fk is None or wk is None:
            continue
        out[kind] = {"fetch_kib": fk, "write_kib": wk, "copy_factor_fetch": f_fac, "copy_factor_write": w_fac,
                     "bytes_per_launch": fk * 1024.0 * f_fac + wk * 1024.0 * w_fac,
                     "kernel_source_sha": kernel_source_hash()}
    return {workload: out, "calibration": {"copy_bytes": calib_bytes, "fetch_kib": f_kib, "write_kib": w_kib}}


# kernel kinds of a counter summary: the library's calls and the bandwidth
# references of measure_ceilings
PMC_KINDS = dict(KERNEL_NAMES, copy_probe=r"stream_copy", read_probe=r"stream_read")


def summarize_pmc(paths) -> str:
    """Per kernel kind, the average over its dispatches of every counter in
    the files (rocprofv3 --pmc counter_collection.csv), and what follows from
    them: the L2's average read and write latency to memory (cycles per
    request in flight), the share of L2 cycles its requests spent stalled for
    want of DRAM credits, the share of 32-byte read and 64-byte write
    requests, and the bytes a dispatch moved per microsecond under counters."""
    import csv
    import re

    vals, durs = {}, {}
    for path in paths:
        for r in csv.DictReader(open(path)):
            kind = next((k for k, rx in PMC_KINDS.items() if re.search(rx, r.get("Kernel_Name", ""))), None)
            if kind is None:
                continue
            vals.setdefault(kind, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            if r.get("Start_Timestamp") and r.get("End_Timestamp"):
                key = (path, r["Dispatch_Id"])
                durs.setdefault(kind, {})[key] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
    lines = []
    for kind in PMC_KINDS:
        if kind not in vals:
            continue
        avg = {k: sum(v) / len(v) for k, v in vals[kind].items()}
        d = list(durs.get(kind, {}).values())
        lines.append(f"### {kind}: {max(len(v) for v in vals[kind].values())} dispatches"
                     + (f", {sum(d) / len(d):.1f} us average under counters" if d else ""))
        lines.append("| counter | average per dispatch |")
        lines.append("|---|---:|")
        for k in sorted(avg):
            lines.append(f"| {k} | {avg[k]:.6g} |")

        def ratio(a, b):
            return avg[a] / avg[b] if a in avg and b in avg and avg[b] else None

        derived = {
            "read latency (L2 cycles per request)": ratio("TCC_EA0_RDREQ_LEVEL_sum", "TCC_EA0_RDREQ_sum"),
            "write latency (L2 cycles per request)": ratio("TCC_EA0_WRREQ_LEVEL_sum", "TCC_EA0_WRREQ_sum"),
            "read DRAM-credit stall share of L2 cycles": ratio("TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum", "TCC_CYCLE_sum"),
            "write DRAM-credit stall share of L2 cycles": ratio("TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum", "TCC_CYCLE_sum"),
            "write stall share of L2 cycles": ratio("TCC_EA0_WRREQ_STALL_sum", "TCC_CYCLE_sum"),
            "32-byte share of read requests": ratio("TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_sum"),
            "64-byte share of write requests": ratio("TCC_EA0_WRREQ_64B_sum", "TCC_EA0_WRREQ_sum"),
            "L2 hit share": (avg["TCC_HIT_sum"] / (avg["TCC_HIT_sum"] + avg["TCC_MISS_sum"])
                             if "TCC_HIT_sum" in avg and "TCC_MISS_sum" in avg and
                             avg["TCC_HIT_sum"] + avg["TCC_MISS_sum"] else None),
            "vector memory latency (cycles per instruction in flight)": ratio("SQ_INST_LEVEL_VMEM", "SQ_INSTS_VMEM"),
        }
        for k, v in derived.items():
            if v is not None:
                lines.append(f"| *{k}* | {v:.4g} |")
        lines.append("")
    return "\n".join(lines)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SRC:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def event_stride(step_s: Optional[float], records: int) -> int:
    """Every stride-th timed step carries `records` timing events (one at its
    start and one after each call), so that the events cost at most
    EVENT_BUDGET of the timed region: a launch-bound step of tens of
    microseconds would otherwise be slowed by its own events, while a step of
    a few milliseconds or more carries them on every step."""
    if not step_s or step_s <= 0:
        return 1
    return max(1, math.ceil(records * EVENT_RECORD_US * 1e-6 / (EVENT_BUDGET * step_s)))


def single_pass_for(w, update: str) -> bool:
    if update == "single-pass" and w.max_norm > 0.0:
        raise SystemExit(f"{w.name} clips at {w.max_norm}: the single pass needs the norm before the update")
    return update == "single-pass" or (update == "auto" and w.max_norm == 0.0)


def bytes_model(w, single: bool = False) -> dict:
    """Algorithmic HBM bytes per parameter of each call kind in one step of
    the fused sequence: micro-steps 1 .. a-1 of every replica per launch, then
    either the last micro-step fused with the replica average followed by the
    update (two passes: g_bar is written and read back), or the last
    micro-step, the average and the update in one pass (g_bar never stored)."""
    sg, sp = 2.0, 2.0
    per = {}
    last = 1 if w.partials else w.a
    if last >= 2:
        per["accumulate_first"] = w.n * (sg + 4.0)
    if last >= 3:
        per["accumulate"] = w.n * (last - 2) * (sg + 8.0)
    sources = w.n * (sg + (4.0 if last >= 2 else 0.0))
    if single:
        per["reduce_adamw"] = sources + 12.0 + 12.0 + sp
    else:
        per["accumulate_reduce"] = sources + 4.0
        per["adamw"] = 16.0 + 12.0 + sp
    return per


def unfused_bytes_per_param(w) -> float:
    """Compulsory bytes per parameter of the step done as separate passes:
    every micro-step a read-modify-write of its accumulator, the replica
    average reading the accumulators and writing g_bar, the update reading
    g_bar once (with n = 1, g_bar is the accumulator; incoming partials are
    read once).  The step time against these bytes is the bandwidth an
    unfused implementation would need to match it."""
    sg = 2.0
    if w.partials:
        return w.n * sg + 4.0 + 30.0
    if w.n == 1:
        return w.a * (sg + 8.0) + 26.0
    return w.n * w.a * (sg + 8.0) + 4.0 + 30.0


def launch_bytes(w, kind: str, single: bool = False) -> float:
    """Algorithmic bytes of one launch of `kind` over the whole flat space."""
    per = bytes_model(w, single)
    launches = {"accumulate": max(1, (1 if w.partials else w.a) - 2)}
    return w.P * per[kind] / launches.get(kind, 1)


def measure_checkpoint(d, directory: str) -> dict:
    """Save the state (current bank of master, m, v and the parameters) as 8
    shards and commit, then restore it as 4 shards; rates in state bytes per
    second, device memory to files and back."""
    import torch

    os.makedirs(directory, exist_ok=True)
    P = d.P
    state_bytes = P * (12 + 2)
    cut = lambda k: [(P * i // k, P * (i + 1) // k) for i in range(k)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    d.save_checkpoint(directory, 1, ranges=cut(8))
    t_save = time.perf_counter() - t0
    t0 = time.perf_counter()
    d.load_checkpoint(directory, ranges=cut(4))
    torch.cuda.synchronize()
    t_load = time.perf_counter() - t0
    return {"metric": "checkpoint save (8 shards) and restore (4 shards) of the step's state",
            "state_bytes": state_bytes, "save_s": t_save, "load_s": t_load,
            "save_gbps": state_bytes / t_save / 1e9, "load_gbps": state_bytes / t_load / 1e9, "unit": "GB/s"}


PEAK_PCIE_GBPS = 2 * 63.0  # PCIe 5.0 x16, both directions (32 GT/s, 128b/130b)


def measure_pcie_copies(nbytes: int = 1 << 30, reps: int = 5) -> dict:
    """Plain copies between pinned host memory and HBM, one direction at a
    time and both at once on two streams: the practical PCIe ceiling the
    offloaded update is held to."""
    import torch

    h_in = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    h_out = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    d_in = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    d_out = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()

    def run(h2d: bool, d2h: bool) -> float:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            if h2d:
                with torch.cuda.stream(s1):
                    d_in.copy_(h_in, non_blocking=True)
            if d2h:
                with torch.cuda.stream(s2):
                    h_out.copy_(d_out, non_blocking=True)
        torch.cuda.synchronize()
        return (int(h2d) + int(d2h)) * nbytes * reps / (time.perf_counter() - t0) / 1e9

    run(True, True)
    return {"h2d_gbps": run(True, False), "d2h_gbps": run(False, True), "both_gbps": run(True, True)}


def measure_ceilings(nbytes: int = 4 << 30, reps: int = 10) -> dict:
    """Bandwidth references measured live on this GPU, in the same process
    (machines differ by a few percent): a copy and a read by one-shot wave64
    kernels shaped like the library's (16 bytes per lane, nontemporal), and
    the HIP runtime's own device-to-device copy (torch ``copy_``), which is
    slower and no ceiling.  The source holds random bytes: HBM moves a
    constant fill 2-4% faster than the random values the workloads carry."""
    import torch

    import benchprobe

    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=gen)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream().cuda_stream

    def timed(fn) -> float:
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    t_copy = timed(lambda: benchprobe.stream("copy", src.data_ptr(), dst.data_ptr(), nbytes, s))
    t_read = timed(lambda: benchprobe.stream("read", src.data_ptr(), 0, nbytes, s))
    t_rt = timed(lambda: dst.copy_(src))
    del src, dst
    torch.cuda.empty_cache()
    return {"copy_gbps": 2 * nbytes / t_copy / 1e9, "read_gbps": nbytes / t_read / 1e9,
            "runtime_copy_gbps": 2 * nbytes / t_rt / 1e9, "bytes": nbytes,
            "what": "one-shot wave64 copy and read (16 B per lane, nontemporal) of random bytes; runtime copy = torch copy_"}


def mix_spec(w, kind: str) -> Optional[dict]:
    """The streams one launch of `kind` reads and writes per element, as a
    benchprobe mix: 16-bit and binary32 streams read, binary32 and 16-bit
    streams written, and whether the first binary32 stream is updated in
    place."""
    n = w.n
    earlier = not w.partials and w.a >= 2  # the last micro-step adds to accumulators
    if kind == "accumulate":
        return dict(r16=1, r32=1, w32=1, w16=0, rmw=True)
    if kind == "accumulate_reduce":
        return dict(r16=n, r32=n if earlier else 0, w32=1, w16=0, rmw=False)
    if kind == "adamw":
        return dict(r16=0, r32=4, w32=3, w16=1, rmw=False)
    if kind == "reduce_adamw" and (not earlier or n <= 13):
        return dict(r16=n, r32=3 + (n if earlier else 0), w32=3, w16=1, rmw=False)
    return None


def measure_mix(w, kind: str, reps: int = 10, max_elems: int = 1 << 29) -> Optional[dict]:
    """The bandwidth the stream mix of `kind` reaches on this GPU: the same
    arrays, access shape and hints as the library's kernel with no arithmetic
    beyond a sum (benchprobe.mix), over min(P, 2^29) elements of random data
    in the workload's value ranges (16-bit streams: bf16 of N(0, 1e-4);
    binary32 streams: N(0, 0.02)); the better of two shapes, with and without
    the staggered start of the library's table-driven kernels."""
    import torch

    import benchprobe

    spec = mix_spec(w, kind)
    if spec is None:
        return None
    N = min(w.P, max_elems) // 256 * 256
    if N == 0:
        return None
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1)
    r16 = [(torch.randn(N, generator=gen, device="cuda") * 1e-4).to(torch.bfloat16) for _ in range(spec["r16"])]
    r32 = [torch.randn(N, generator=gen, device="cuda") * 0.02 for _ in range(spec["r32"])]
    w32 = ([r32[0]] if spec["rmw"] else []) + [torch.empty(N, device="cuda")
                                               for _ in range(spec["w32"] - (1 if spec["rmw"] else 0))]
    w16 = [torch.empty(N, dtype=torch.int16, device="cuda") for _ in range(spec["w16"])]
    stag = torch.zeros(N // 16384 + 1, dtype=torch.int64, device="cuda")
    addr = lambda ts: [t.data_ptr() for t in ts]  # noqa: E731
    st = torch.cuda.current_stream()
    per = 2 * spec["r16"] + 4 * spec["r32"] + 4 * spec["w32"] + 2 * spec["w16"]
    shapes = {}
    for shape, sp in (("plain", 0), ("staggered", stag.data_ptr())):
        def once():
            benchprobe.mix(addr(r16), addr(r32), addr(w32), addr(w16), N, st.cuda_stream, rmw=spec["rmw"],
                           stagger=sp)

        once()
        once()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            once()
        e1.record(st)
        torch.cuda.synchronize()
        shapes[shape] = per * N / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9
    gbps = max(shapes.values())
    del r16, r32, w32, w16, stag
    torch.cuda.empty_cache()
    return {"mix": {k: v for k, v in spec.items()}, "bytes_per_elem": per, "elements": N, "gbps_by_shape": shapes,
            "gbps": gbps, "frac": gbps / PEAK_HBM_GBPS}


def run_gpu(w, steps: int, warmup: int, chunk: int = 0, calib: int = 0, bind: str = "flat", single: bool = False,
            ckpt_dir: str = "", state: str = "hbm", graph: bool = False, offload: str = "direct",
            layout: str = "auto", log_path: str = "", spacer: int = 0):
    import torch

    import synth
    from gradient_reduce_adam_amd import DP_ROLE_GRAD, dp_plan_bind_flat, driver

    torch.cuda.set_device(0)
    # an allocation held ahead of the state moves the state to other HBM pages
    spacer_buf = torch.empty(spacer, dtype=torch.uint8, device="cuda") if spacer else None
    if calib:
        src = torch.empty(calib, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    d = driver.DPStep(w.numel, w.n, w.a, w.grad_dtype, w.param_dtype, lr=w.lr, eps=w.eps,
                      weight_decay=w.weight_decay, beta1=w.beta1, beta2=w.beta2, max_norm=w.max_norm,
                      scaler=w.scaler, init_scale=w.init_scale, backoff=w.backoff, growth=w.growth,
                      growth_interval=w.growth_interval, partials=w.partials, chunk_elems=chunk, single_pass=single,
                      state_location=state, stream=torch.cuda.Stream() if graph else None, offload=offload,
                      layout=layout)
    st_obj = d.stream
    stream = st_obj.cuda_stream
    d.set_master(lambda ptr: synth.master_device(w, ptr, stream))
    if bind == "tensors":
        # the same buffers, bound through per-tensor pointer tables
        off = [int(x) for x in w.offsets[:-1]]

        def per_tensor(t):
            return [t.data_ptr() + o * t.element_size() for o in off]

        for b, (w_, m_, v_) in enumerate(d.banks):
            for role, t in (("master", w_), ("exp_avg", m_), ("exp_avg_sq", v_)):
                d.plan.bind_tensors(role, per_tensor(t), b)
        d.plan.bind_tensors("param", per_tensor(d.param))
        for r, t in enumerate(d.acc):
            d.plan.bind_tensors("acc", per_tensor(t), r)
        if d.gbar is not None and not (w.n == 1 and not w.partials):
            d.plan.bind_tensors("gbar", per_tensor(d.gbar))

    # one batch of gradients, resident before the timed region
    calls = [(r, 1) for r in range(w.n)] if w.partials else [(r, k) for k in range(1, w.a + 1) for r in range(w.n)]
    per_buf = 2 * w.P
    # a ring of distinct buffers; a micro-step's n replicas (and consecutive
    # launches) never share one, and every buffer is far larger than the caches
    free, _ = torch.cuda.mem_get_info()
    budget = min(RESIDENT_GRAD_BUDGET, free - 4e9)  # leave room for the library's tables and torch
    nbuf = len(calls) if len(calls) * per_buf <= budget else int(budget // per_buf)
    nbuf = max(nbuf, 2 * w.n if not w.partials else w.n)
    # one allocation; a micro-step's n replicas take consecutive rows
    ring = torch.empty((nbuf, w.P), dtype=torch.int16, device="cuda")
    bufs = list(ring.unbind(0))
    addr = {}
    for i, (r, k) in enumerate(calls):
        b = bufs[i % nbuf]
        if i < nbuf:
            synth.grad_device(w.with_(injections=()), 1, r, k, b.data_ptr(), d.scale, stream)
        addr[(r, k)] = b.data_ptr()
    torch.cuda.synchronize()

    plan = d.plan
    off_bytes = [2 * int(x) for x in w.offsets[:-1]]

    def bind_grad(r, a):
        # flat: one base per replica; tensors and grads: one pointer per tensor, a new
        # table before every micro-step as a framework with per-tensor
        # gradient buffers would bind them
        if bind in ("tensors", "grads"):
            plan.bind_tensors("grad", [a + o for o in off_bytes], r)
        else:
            dp_plan_bind_flat(plan.handle, DP_ROLE_GRAD, r, a)

    last = 1 if w.partials else w.a
    ncalls = (last - 1) + (1 if single else 3)

    def one_step(marks=None):
        """Issues one step.  With `marks` (ncalls + 1 events) it records
        marks[0] at the start and marks[i + 1] after call i, so call i is timed
        from marks[i] to marks[i + 1] and the step from the first to the last.
        Returns the kinds of the calls in order."""
        kinds = []

        def call(kind, fn):
            fn()
            kinds.append(kind)
            if marks is not None:
                marks[len(kinds)].record(st_obj)

        if marks is not None:
            marks[0].record(st_obj)
        for k in range(1, last):
            for r in range(w.n):
                bind_grad(r, addr[(r, k)])
            call("accumulate_first" if k == 1 else "accumulate",
                 lambda k=k: plan.accumulate_all(first=(k == 1), stream=stream))
        for r in range(w.n):
            bind_grad(r, addr[(r, last)])
        if single:  # one call: the single-pass kernel, the statistics fold and the (idle) parameter restore
            call("reduce_adamw", lambda: plan.reduce_adam_step(w.lr, w.eps, w.weight_decay, stream=stream))
            return kinds
        call("accumulate_reduce", lambda: plan.accumulate_reduce(stream=stream))
        call("finalize", lambda: plan.grad_stats(scan=False, max_norm=w.max_norm, stream=stream))
        if d.offload == "staged":
            call("adamw", d.staged_update)
        else:
            call("adamw", lambda: plan.adam_step(w.lr, w.eps, w.weight_decay, stream=stream))
        return kinds

    def new_marks():
        return [torch.cuda.Event(enable_timing=True) for _ in range(ncalls + 1)]

    # warm-up, each step timed on the host: the shortest sets the event stride
    warm_s = []
    for _ in range(warmup):
        t0 = time.perf_counter()
        one_step()
        torch.cuda.synchronize()
        warm_s.append(time.perf_counter() - t0)
    stride = event_stride(min(warm_s) if warm_s else None, ncalls + 1)
    marks = {i: new_marks() for i in range(0, steps, stride)}
    for m in marks.values():  # each event created and recorded once before the timed region
        for e in m:
            e.record(st_obj)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        kinds = one_step(marks.get(i))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_ms = sorted(m[0].elapsed_time(m[-1]) for m in marks.values())
    events = {}
    for m in marks.values():
        for j, kind in enumerate(kinds):
            events.setdefault(kind, []).append((m[j], m[j + 1]))
    skipped_ms = None
    if w.injections and not graph:
        # one step whose g_bar holds an inf, as the workload injects one: the
        # step is skipped (single pass: computed, then discarded and the
        # parameters emitted again); the buffer is restored afterwards
        _, r0, _, idx, val = w.injections[0]
        ptr = addr[(r0 % w.n, last)] + 2 * idx
        flat = ring.view(-1)
        pos = (ptr - ring.data_ptr()) // 2
        saved = flat[pos].clone()
        torch.cuda.synchronize()
        synth._poke_u16(ptr, synth._lp_bits(val, w.grad_dtype), stream)
        m = new_marks()
        one_step(m)
        torch.cuda.synchronize()
        skipped_ms = m[0].elapsed_time(m[-1])
        assert d.read_state()["found_inf"] == 1
        flat[pos] = saved
        torch.cuda.synchronize()
    if graph:  # the same step as one HIP graph: capture, warm up, time the replays
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st_obj):
            one_step()
        # replayed on the step's stream, like the eager steps (torch replays
        # on the current stream)
        with torch.cuda.stream(st_obj):
            for _ in range(warmup):
                g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(st_obj):
            for _ in range(steps):
                g.replay()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    state = d.read_state()
    if log_path:  # per-step records, outside everything timed above
        with open(log_path, "w") as f:
            for _ in range(steps):
                m = new_marks()
                kinds = one_step(m)
                s_ = d.read_state()  # synchronises the stream
                ms = {}
                for j, kind in enumerate(kinds):
                    ms[kind] = ms.get(kind, 0.0) + m[j].elapsed_time(m[j + 1])
                f.write(json.dumps({"workload": w.name, "t": s_["t"], "iter": s_["iter"], "found_inf": s_["found_inf"],
                                    "scale": s_["scale"], "norm": s_["norm"], "clip": s_["clip"], "call_ms": ms,
                                    "step_ms": sum(ms.values()),
                                    "params_per_s": w.P / (sum(ms.values()) * 1e-3)}) + "\n")
    ckpt = measure_checkpoint(d, ckpt_dir) if ckpt_dir else None
    per_kind = {}
    for kind, pairs in events.items():
        ms = [a.elapsed_time(b) for a, b in pairs]
        per_kind[kind] = {"launches": len(ms), "avg_ms": sum(ms) / len(ms), "total_ms": sum(ms)}
    used_layout = d.layout
    d.close()
    del bufs, ring, spacer_buf
    torch.cuda.empty_cache()
    per_kind["skipped_step_ms"] = skipped_ms
    per_kind["step_ms"] = None if graph else step_ms  # the instrumented eager steps; a graph replays them as one
    per_kind["event_stride"] = stride
    per_kind["instrumented_steps"] = len(marks)
    return elapsed, per_kind, state, ckpt, used_layout


def run_overlap(w, steps: int, warmup: int, bucket_mbs, tokens: int, single: bool = False, micro: bool = False):
    """The bucketed reduction overlapped with a synthetic backward pass; with
    single, each bucket's reduction also updates its parameters (the single
    pass in buckets); with micro, the earlier micro-steps' accumulation is
    bucketed and overlapped too."""
    import torch

    import benchprobe
    import synth
    from gradient_reduce_adam_amd import driver

    torch.cuda.set_device(0)
    d = driver.DPStep(w.numel, w.n, w.a, w.grad_dtype, w.param_dtype, lr=w.lr, eps=w.eps,
                      weight_decay=w.weight_decay, beta1=w.beta1, beta2=w.beta2, max_norm=w.max_norm,
                      scaler=w.scaler, init_scale=w.init_scale, backoff=w.backoff, growth=w.growth,
                      growth_interval=w.growth_interval, partials=w.partials, single_pass=single)
    st = d.stream.cuda_stream
    d.set_master(lambda ptr: synth.master_device(w, ptr, st))
    wi = w.with_(injections=())
    slots = [torch.empty(w.P, dtype=torch.int16, device="cuda") for _ in range(w.n)]
    addrs = [t.data_ptr() for t in slots]

    def produce(step, k, lo, hi, stream):
        benchprobe.backward_bucket(wi, step, k, lo, hi, addrs, d.scale, stream, tokens)

    def timed(fn, reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(d.stream)
        for _ in range(reps):
            fn()
        e1.record(d.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    # the two parts alone, each after one untimed call: one micro-step's
    # backward, and the last micro-step's reduction
    last = 1 if w.partials else w.a
    produce(1, last, 0, w.P, st)
    t_bwd = timed(lambda: produce(1, last, 0, w.P, st), 3)
    for r, a_ in enumerate(addrs):
        driver.dp_plan_bind_flat(d.plan.handle, driver.DP_ROLE_GRAD, r, a_)
    reds = []
    for _ in range(4):  # the last micro-step's reduction as the step issues it (after earlier micro-steps)
        if last > 1:
            d.plan.accumulate_all(first=True, stream=st)
        if single:  # the reduction, the statistics and the update in one pass
            reds.append(timed(lambda: d.plan.reduce_adam_step(w.lr, w.eps, w.weight_decay, stream=st), 1))
        else:
            reds.append(timed(lambda: d.plan.accumulate_reduce(stream=st), 1))
    t_red = statistics.median(reds[1:])
    d.close()
    del d
    torch.cuda.empty_cache()
    rs = torch.cuda.Stream()
    lines = []
    for mb in bucket_mbs:
        # incoming partials arrive from the exchange in pieces: their buckets
        # may cut tensors; a backward pass finishes whole tensors
        buckets = driver.backward_buckets(w.numel, int(mb * (1 << 20)), split=w.partials)
        res, last_ms = {}, {}
        for mode in ("sequential", "overlapped"):
            d = driver.DPStep(w.numel, w.n, w.a, w.grad_dtype, w.param_dtype, lr=w.lr, eps=w.eps,
                              weight_decay=w.weight_decay, beta1=w.beta1, beta2=w.beta2, max_norm=w.max_norm,
                              scaler=w.scaler, init_scale=w.init_scale, backoff=w.backoff, growth=w.growth,
                              growth_interval=w.growth_interval, partials=w.partials, single_pass=single)
            d.set_master(lambda ptr: synth.master_device(w, ptr, d.stream.cuda_stream))
            marks = []

            def step():
                m = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                marks.append(m)
                d.step_overlapped(addrs, produce, buckets, reduce_stream=rs if mode == "overlapped" else None,
                                  sync_scale=False, marks=m, micro_buckets=micro)

            for _ in range(warmup):
                step()
            del marks[:]
            res[mode] = timed(step, steps)
            last_ms[mode] = sum(a.elapsed_time(b) for a, b in marks) / len(marks)
            d.close()
            del d
            torch.cuda.empty_cache()
        saved = last_ms["sequential"] - last_ms["overlapped"]
        what = "replica reduction and update" if single else "replica reduction"
        lines.append({"metric": f"last micro-step (synthetic backward + {what}) with the {what} "
                                "in buckets, sequential and overlapped on a second stream", "unit": "ms",
                      "config": {"workload": w.name, "bucket_mb": mb, "buckets": len(buckets), "tokens": tokens,
                                 "buckets_cut_tensors": bool(w.partials),
                                 "update": "single-pass" if single else "two-pass",
                                 "micro_steps_bucketed": bool(micro)},
                      "last_micro_step_sequential_ms": last_ms["sequential"],
                      "last_micro_step_overlapped_ms": last_ms["overlapped"], "saved_ms": saved,
                      "step_sequential_ms": res["sequential"], "step_overlapped_ms": res["overlapped"],
                      "backward_ms_per_micro_step": t_bwd, "reduce_ms": t_red,
                      "hidden_frac_of_reduce": saved / t_red})
    del slots
    torch.cuda.empty_cache()
    return lines


# hipDeviceAttribute_t values of the ROCm 7 headers
HIP_ATTR_MEMORY_BUS_WIDTH = 59   # hipDeviceAttributeMemoryBusWidth, bits
HIP_ATTR_MEMORY_CLOCK_RATE = 60  # hipDeviceAttributeMemoryClockRate, kHz


def device_info() -> dict:
    """What the runtime reports about the device: name, compute units, HBM
    size, and the memory clock and bus width.  On MI355X the runtime reports
    a 2 GHz clock for its HBM3E, which moves data at 8 Gb/s per pin: four
    transfers per reported clock, so clock x 4 x width is the interface's
    nominal rate (8.19 TB/s), a cross-check of the published 8 TB/s that
    stays the roofline's denominator."""
    import ctypes

    import torch

    dev = torch.cuda.current_device()
    pr = torch.cuda.get_device_properties(dev)
    info = {"name": pr.name, "arch": pr.gcnArchName, "compute_units": pr.multi_processor_count,
            "hbm_bytes": pr.total_memory, "mem_clock_khz": None, "mem_bus_bits": None, "nominal_gbps": None}
    with open("/proc/self/maps") as f:
        path = next((ln.split()[-1] for ln in f if "libamdhip64" in ln), None)
    if path:
        hip = ctypes.CDLL(path)
        v = ctypes.c_int()
        if hip.hipDeviceGetAttribute(ctypes.byref(v), HIP_ATTR_MEMORY_BUS_WIDTH, dev) == 0:
            info["mem_bus_bits"] = v.value
        if hip.hipDeviceGetAttribute(ctypes.byref(v), HIP_ATTR_MEMORY_CLOCK_RATE, dev) == 0:
            info["mem_clock_khz"] = v.value
        if info["mem_bus_bits"] and info["mem_clock_khz"]:
            info["nominal_gbps"] = info["mem_clock_khz"] * 1e3 * 4 * info["mem_bus_bits"] / 8 / 1e9
    return info


def cpu_share(cgroup_cpu_max: str = "/sys/fs/cgroup/cpu.max") -> dict:
    """The host threads this process may use: the cores of its affinity mask,
    capped by a cgroup CPU quota and by OMP_NUM_THREADS where either is set
    (a machine shared between GPUs gives each GPU's jobs a share of its
    cores)."""
    affinity = len(os.sched_getaffinity(0))
    quota = None
    try:
        with open(cgroup_cpu_max) as f:
            q, period = f.read().split()[:2]
        if q != "max":
            quota = max(1, int(math.ceil(int(q) / int(period))))
    except (OSError, ValueError):
        pass
    omp = os.environ.get("OMP_NUM_THREADS", "")
    omp_n = int(omp) if omp.isdigit() and int(omp) > 0 else None
    share = min(x for x in (affinity, quota, omp_n) if x is not None)
    return {"affinity_cores": affinity, "cgroup_quota_cores": quota, "omp_num_threads": omp_n, "threads": share}


def cpu_baseline(w, sample: int) -> dict:
    """The oracle, as it stands, on a bounded sample of the same workload:
    whole steps (every micro-step, the replica tree, the statistics and the
    update) over `sample` parameters in one tensor, on one batch of gradients
    generated beforehand (not timed).  Timed twice: on one thread, and on
    every thread of the process's CPU share; each leg repeats steps until
    about CPU_BASELINE_SECONDS of oracle work are timed.  The oracle's driver
    spreads the accumulation, the replica tree and the statistics over its
    threads and runs the update of a window on one, so the second leg gains
    on the first only in those parts."""
    import oracle
    import synth

    share = cpu_share()
    gen_threads = share["threads"]
    ws = w.with_(numel=(sample,), injections=(), scaled_tensors=())
    calls = [(r, 1) for r in range(ws.n)] if ws.partials else [(r, k) for k in range(1, ws.a + 1) for r in range(ws.n)]
    scale = ws.init_scale if ws.scaler != "none" else 1.0
    pre = {rk: synth.grad_host(ws, 1, rk[0], rk[1], 0, sample, scale, threads=gen_threads) for rk in calls}
    master = synth.master_host(ws, 0, sample, threads=gen_threads)

    def grad_fn(step, r, k, lo, hi, sc):
        return pre[(r, k)][lo:hi]

    def leg(threads: int) -> dict:
        # runs of steps until the time is reached
        steps, dt, k = 0, 0.0, 1
        while dt < CPU_BASELINE_SECONDS:
            t0 = time.perf_counter()
            oracle.run(ws, k, grad_fn, lambda lo, hi: master[lo:hi], threads=threads, chunk=1 << 18)
            dt += time.perf_counter() - t0
            steps += k
            k = max(1, min(200, int(math.ceil((CPU_BASELINE_SECONDS - dt) * steps / dt))))
        return {"value": sample * steps / dt, "cores": threads, "steps": steps, "seconds": dt}

    # one untimed step first (pages of the inputs and the state touched once)
    oracle.run(ws, 1, grad_fn, lambda lo, hi: master[lo:hi], threads=gen_threads, chunk=1 << 18)
    one = leg(1)
    many = leg(gen_threads) if gen_threads > 1 else one
    return {"value": many["value"], "unit": "params/s", "cores": many["cores"], "kind": "oracle",
            "sample": f"{many['steps']} full steps of {ws.name} (n={ws.n}, a={ws.a}: every micro-step, the replica "
                      f"tree, statistics and update) over {sample} params in one tensor on one pre-generated batch, "
                      f"{many['seconds']:.1f} s on {many['cores']} threads; the same on 1 thread: {one['steps']} "
                      f"steps in {one['seconds']:.1f} s",
            "one_thread": {"value": one["value"], "unit": "params/s", "cores": 1, "steps": one["steps"],
                           "seconds": one["seconds"]},
            "host": share}


def zero3_single_pass(steps: int, warmup: int, placements: int) -> dict:
    """The ZeRO-3 rank share's single pass (8 incoming bf16 partials, dynamic
    loss scale) timed in this process at several HBM placements: its arrays
    allocated behind a spacer of 0, 3, 6, ... GiB.  Its bandwidth depends on
    where its 15 concurrent streams land in physical memory, so one placement
    is not its figure: the median and the range are."""
    from synth import workloads

    w = workloads.by_name("zero3_rank_7b")
    per_param = bytes_model(w, True)
    runs = []
    for k in range(placements):
        elapsed, per_kind, _, _, _ = run_gpu(w, steps, warmup, single=True, spacer=k * (3 << 30))
        ms = elapsed * 1e3 / steps
        k_ms = per_kind["reduce_adamw"]["avg_ms"]
        k_gbps = launch_bytes(w, "reduce_adamw", True) / (k_ms * 1e-3) / 1e9
        runs.append({"spacer_gib": 3 * k, "ms_per_step": ms, "params_per_s": w.P / (ms * 1e-3),
                     "hbm_gbps": sum(per_param.values()) * w.P / (ms * 1e-3) / 1e9,
                     "reduce_adamw_ms": k_ms, "reduce_adamw_gbps": k_gbps, "frac": k_gbps / PEAK_HBM_GBPS,
                     "skipped_step_ms": per_kind.get("skipped_step_ms")})
    fr = sorted(r["frac"] for r in runs)
    med = statistics.median(r["ms_per_step"] for r in runs)
    ceiling = measure_mix(w, "reduce_adamw")
    if ceiling:
        ceiling["library_of_ceiling_median"] = statistics.median(r["reduce_adamw_gbps"] for r in runs) / ceiling["gbps"]
    return {"workload": w.name, "mix_ceiling": ceiling, "params": w.P, "update": "single-pass", "steps": steps,
            "bytes_per_param_step": sum(per_param.values()),
            "ms_per_step_median": med, "params_per_s_median": w.P / (med * 1e-3),
            "hbm_gbps_median": sum(per_param.values()) * w.P / (med * 1e-3) / 1e9,
            "reduce_adamw_frac_median": statistics.median(fr), "reduce_adamw_frac_range": [fr[0], fr[-1]],
            "placements": runs}


def progress(msg: str) -> None:
    """A progress line on stderr (the JSON line is the only stdout)."""
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the n replicas share its HBM and there is no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    from synth import workloads

    if args.summarize_pmc:
        print(summarize_pmc(args.summarize_pmc))
        return
    if args.summarize_counters:
        res = summarize_counters(*args.summarize_counters, args.workload, args.copy_calibration)
        old = {}
        if os.path.exists(TRAFFIC_FILE):
            with open(TRAFFIC_FILE) as f:
                old = json.load(f)
        old.update(res)
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(old, f, indent=1)
        print(json.dumps(res, indent=1))
        return
    w = workloads.by_name(args.workload)
    single = single_pass_for(w, args.update)
    if args.overlap:
        for line in run_overlap(w, args.steps, args.warmup, [float(x) for x in args.overlap.split(",")],
                                args.tokens, single, args.micro_buckets):
            print(json.dumps(line), flush=True)
        return
    progress(f"{w.name}: {args.warmup} warm-up and {args.steps} timed steps ({'single' if single else 'two'}-pass)")
    elapsed, per_kind, state, ckpt, layout = run_gpu(w, args.steps, args.warmup, args.chunk, args.copy_calibration,
                                                     args.bind, single, args.checkpoint_dir, args.state, args.graph,
                                                     args.offload, args.layout, args.log_steps)
    ms_per_step = elapsed * 1e3 / args.steps
    per_param = bytes_model(w, single)
    step_bytes = sum(per_param.values()) * w.P
    hbm_gbps = step_bytes / (ms_per_step * 1e-3) / 1e9

    skipped_ms = per_kind.pop("skipped_step_ms", None)
    step_ms = per_kind.pop("step_ms", None)
    stride = per_kind.pop("event_stride", None)
    instrumented = per_kind.pop("instrumented_steps", None)
    # dominant kernel: the call kind that moves the most algorithmic bytes per step
    dom = max(per_param, key=lambda k: per_param[k])
    dom_bytes = launch_bytes(w, dom, single)
    dom_ms = per_kind[dom]["avg_ms"]
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        ent = t.get(w.name, {}).get(dom)
        if ent and ent.get("kernel_source_sha") == kernel_source_hash():
            traffic = ent["bytes_per_launch"]
    progress("measured ceilings (copy and read of random bytes, and the stream mixes of the main kernels)")
    mix = {}
    if args.state == "hbm":
        for kind in [k for k in per_param if k in per_kind]:
            m = measure_mix(w, kind)
            if m:
                lib_gbps = launch_bytes(w, kind, single) / (per_kind[kind]["avg_ms"] * 1e-3) / 1e9
                m["library_gbps"] = lib_gbps
                m["library_of_ceiling"] = lib_gbps / m["gbps"]
                mix[kind] = m

    line = {
        "metric": "params updated/sec and achieved HBM GB/s (% of peak) per full DP step",
        "value": w.P * args.steps / elapsed,
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "params": w.P, "tensors": w.T, "n_replicas": w.n, "micro_steps": w.a,
                   "grad_dtype": w.grad_dtype, "param_dtype": w.param_dtype, "state": "fp32 master/m/v",
                   "update_arithmetic": "f64", "clip": w.max_norm, "loss_scale": w.scaler,
                   "global_batch": 4 * w.n * w.a, "parallelism": "dp (replicas in one GPU's HBM)",
                   "chunk_elems": args.chunk or 16384, "binding": args.bind,
                   "update": "single-pass" if single else "two-pass",
                   "launch": "hip graph replay" if args.graph else "eager", "layout": layout},
        "hbm_gbps": hbm_gbps,
        "hbm_frac": hbm_gbps / PEAK_HBM_GBPS,
        "bytes_per_param_step": sum(per_param.values()),
        "unfused_bytes_per_param_step": unfused_bytes_per_param(w),
        "unfused_equiv_gbps": unfused_bytes_per_param(w) * w.P / (ms_per_step * 1e-3) / 1e9,
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic, "bytes_per_launch": dom_bytes,
                     "avg_launch_ms": dom_ms,
                     "traffic_source": ("FETCH_SIZE + WRITE_SIZE per launch from a separate rocprofv3 --pmc run of "
                                        "this workload (profiles/traffic.json), scaled by the same counters on a "
                                        "plain copy; valid for the kernel source it was taken on (hash checked)"
                                        if traffic is not None else None)},
        # per-call times of the eager timed steps that carried events
        "breakdown_ms_per_step": {k: v["total_ms"] / instrumented for k, v in per_kind.items()},
        "event_stride": stride,
        "instrumented_steps": instrumented,
        "final_state": {"t": state["t"], "norm": state["norm"], "found_inf": state["found_inf"]},
        "skipped_step_ms": skipped_ms,
        # per-step event times of the timed steps: the median and the fastest
        "step_ms_median": statistics.median(step_ms) if step_ms else None,
        "step_ms_min": step_ms[0] if step_ms else None,
        "device": device_info(),
        "measured_ceilings": dict(measure_ceilings(), stream_mixes=mix),
        "cpu_baseline": None,
    }
    if args.state == "host":
        # the offload variant: the update is bound by PCIe, which carries the
        # state both ways (12 B/param read, 12 B/param written)
        upd = "reduce_adamw" if single else "adamw"
        upd_ms = per_kind[upd]["avg_ms"]
        line["metric"] = "params updated/sec per full DP step, optimizer state in pinned host memory"
        line["config"]["state_location"] = ("host (pinned, read and written by the update kernels over PCIe)"
                                            if args.offload == "direct" else
                                            "host (pinned, copied through device slots on two copy streams)")
        line["pcie_copies"] = measure_pcie_copies()
        line["roofline"] = {"kernel": upd, "bound": "pcie", "achieved": 24.0 * w.P / (upd_ms * 1e-3) / 1e9,
                            "peak": PEAK_PCIE_GBPS, "unit": "GB/s",
                            "frac": 24.0 * w.P / (upd_ms * 1e-3) / 1e9 / PEAK_PCIE_GBPS, "traffic": None,
                            "bytes_per_launch": 24.0 * w.P, "avg_launch_ms": upd_ms}
    if w.name == "unsharded_7b" and args.zero3_placements > 0 and args.state == "hbm" and not args.graph:
        progress(f"ZeRO-3 rank share, single pass, {args.zero3_placements} placements")
        line["zero3_rank_7b_single_pass"] = zero3_single_pass(args.steps, args.warmup, args.zero3_placements)
    if not args.no_cpu_baseline:
        progress(f"CPU baseline: the oracle on {args.cpu_sample} params of {w.name}")
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_sample)
    print(json.dumps(line), flush=True)
    if ckpt:
        ckpt["config"] = {"workload": w.name, "params": w.P}
        print(json.dumps(ckpt), flush=True)


if __name__ == "__main__":
    main()
