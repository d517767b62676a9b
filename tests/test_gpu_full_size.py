"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (default chunk size, the fused step sequence).

Every workload runs for its own number of steps.  The oracle computes the
global statistics of every step over the whole flat range (they decide
clipping and skipping) and the update on sampled windows: the first and last
elements, a window around every tensor boundary (224 of them in the 7B
layout), windows straddling chunk boundaries, windows around every injected
non-finite value, and seeded random windows.  Master, m and v must also lie
within the ulp bound of the comparison (bit-exact without clipping).
Two properties are checked at full size as well: the sum of squares the
library reports is the binary64 sum of squares of its own g_bar (a torch
reduction), and the skip flag is set exactly when that g_bar holds an inf or
NaN."""
import time

import numpy as np
import pytest
import torch

from synth import workloads

from gpu_common import DeviceRun, assert_scalars_match, assert_state_close, log, oracle_run, sample_windows, ulp_bound

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

# every workload at its own step count; the workloads without clipping also
# run through the single pass, as the benchmark times them (the 7B ZeRO-3
# share skips its third step on both paths)
CASES = [("gpt2_small", 20, False), ("zero3_rank_7b", 5, False), ("zero3_rank_7b", 5, True),
         ("unsharded_7b", 3, False), ("unsharded_7b", 3, True), ("tp_column_slice", 3, False)]

# the oracle's run of a workload, shared by its two update paths (same
# windows, same steps): the full statistics pass is the expensive part
_ORACLE = {}


def _oracle(w, steps, wins):
    key = (w.name, steps, tuple(wins))
    if key not in _ORACLE:
        _ORACLE.clear()
        t0 = time.time()
        _ORACLE[key] = oracle_run(w, steps, windows=wins, keep_gbar=(steps,),
                                  progress=lambda s, rec: log(f"  oracle step {s}: norm {rec['norm']:.6g} "
                                                              f"found_inf {rec['found_inf']} ({time.time() - t0:.0f} s)"))
        log(f"  oracle done in {time.time() - t0:.1f} s")
    return _ORACLE[key]


def _sumsq_fp64(x: torch.Tensor) -> float:
    piece = 1 << 27
    tot = torch.zeros((), dtype=torch.float64, device=x.device)
    for i in range(0, x.numel(), piece):
        tot += x[i:i + piece].double().square().sum()
    return float(tot.item())


def _nonfinite(x: torch.Tensor) -> bool:
    piece = 1 << 27
    return any(bool((~torch.isfinite(x[i:i + piece])).any()) for i in range(0, x.numel(), piece))


@pytest.mark.parametrize("name,steps,single", CASES)
def test_full_size_sampled_parity(name, steps, single):
    w = workloads.by_name(name)
    wins = sample_windows(w)
    log(f"full size {name}: P={w.P} T={w.T} n={w.n} a={w.a} steps={steps} single_pass={single} "
        f"windows={len(wins)} ({sum(h - l for l, h in wins)} elements)")
    t0 = time.time()
    run = DeviceRun(w, single_pass=single)
    try:
        states = run.run(steps)
        got = {win: run.window(*win) for win in wins}
        if not single:  # the single pass never stores g_bar
            ss = _sumsq_fp64(run.d.gbar)
            bad = _nonfinite(run.d.gbar)
    finally:
        run.close()
    log(f"  gpu done in {time.time() - t0:.1f} s; last norm {states[-1]['norm']:.6g} clip {states[-1]['clip']:.6g}")
    if not single:
        assert abs(states[-1]["sumsq"] - ss) <= 1e-12 * ss, (states[-1]["sumsq"], ss)
        assert states[-1]["found_inf"] == int(bad)

    ref = _oracle(w, steps, wins)
    assert len(states) == len(ref.scalars) == w.steps
    for s, (g, r) in enumerate(zip(states, ref.scalars), start=1):
        assert_scalars_match(g, r, where=f"{name} step {s}")
    worst = {}
    for win in wins:
        rep = assert_state_close(got[win], ref.state[win], ulp_bound(w), where=f"{name} window {win}")
        for k, v in rep.items():
            worst[k] = max(worst.get(k, 0), v)
        if not single:
            assert np.array_equal(got[win]["gbar"].view(np.uint32), ref.gbar[steps][win].view(np.uint32)), win
    log(f"  max ulp over windows: {worst} (bound {ulp_bound(w)})")


def _device_state(run):
    """master, m, v (of the current bank) and p, as device copies."""
    torch.cuda.synchronize()
    w_, m_, v_ = run.d.state_tensors()
    return [w_.clone(), m_.clone(), v_.clone(), run.d.param.clone()]


@pytest.mark.parametrize("name,steps,single", [("gpt2_small", 2, False), ("zero3_rank_7b", 3, True)])
def test_full_size_buckets_equal_whole(name, steps, single):
    """The bucketed step at full size, as ``bench.py --overlap`` issues it:
    every micro-step's accumulation and the reduction (or the single pass) in
    buckets on a second stream, the producer writing each bucket on the
    step's stream.  State and scalars equal the whole step's bit for bit
    (the ZeRO-3 share's third step is skipped by its injected inf)."""
    from gradient_reduce_adam_amd import driver
    import synth
    w = workloads.by_name(name)
    run = DeviceRun(w, single_pass=single)
    try:
        whole_states = run.run(steps)
        whole = _device_state(run)
    finally:
        run.close()
    buckets = driver.backward_buckets(w.numel, 64 << 20, split=w.partials)
    log(f"full-size buckets {name}: {len(buckets)} buckets of 64 MB, {steps} steps, single_pass={single}")
    run = DeviceRun(w, single_pass=single)
    slots = [torch.empty(w.P, dtype=torch.int16, device="cuda") for _ in range(w.n)]
    addrs = [t.data_ptr() for t in slots]
    d = run.d

    def produce(step, k, lo, hi, stream):
        for r in range(w.n):
            synth.grad_device(w, step, r, k, addrs[r] + 2 * lo, d.scale, stream, lo, hi)

    try:
        rs = torch.cuda.Stream()
        states = [d.step_overlapped(addrs, produce, buckets, reduce_stream=rs, micro_buckets=True)
                  for _ in range(steps)]
        got = _device_state(run)
    finally:
        run.close()
        del slots
    for s, (a, b) in enumerate(zip(states, whole_states), start=1):
        assert np.array_equal(np.array(list(a.values()), np.float64).view(np.uint64),
                              np.array(list(b.values()), np.float64).view(np.uint64)), f"step {s} scalars"
    for k, (x, y) in enumerate(zip(got, whole)):
        assert torch.equal(x.view(torch.int16 if x.element_size() == 2 else torch.int32),
                           y.view(torch.int16 if y.element_size() == 2 else torch.int32)), ("w", "m", "v", "p")[k]
