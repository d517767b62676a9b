"""Random schedules of the bucket calls, on the GPU, through the C ABI.

For each seed, every micro-step is issued whole or as a random partition of
the flat space into buckets (ends at tensor starts or multiples of 256
elements into a tensor), in a random order; the last micro-step goes through
one of the reduction routes (fused whole, fused buckets, or accumulated in
buckets and then reduced from the accumulators in buckets), or, for runs
without clipping, through the single pass whole or in buckets.  Between the
calls, out-of-order calls are tried: each must fail with DP_ERR_STATE or
DP_ERR_INVALID_ARG and change nothing.  The state and scalars after every
schedule equal, bit for bit, those of the plain whole-space step."""
import numpy as np
import pytest
import torch

import gradient_reduce_adam_amd as dp
import synth
from synth import workloads

from gpu_common import DeviceRun, log

pytestmark = pytest.mark.gpu

RAGGED = (3000, 17, 4096, 5, 70001, 256, 1, 65536, 131075)


def _grid(w):
    """Every valid bucket end: tensor starts, multiples of 256 into a tensor, P."""
    off = [int(x) for x in w.offsets]
    ends = set()
    for t in range(w.T):
        ends.update(range(off[t], off[t + 1], 256))
    ends.add(w.P)
    return sorted(ends)


def _partition(rng, grid, P):
    k = int(rng.integers(1, 9))
    cuts = sorted(set([0, P] + [int(x) for x in rng.choice(grid, size=min(k, len(grid)), replace=False)]))
    buckets = [(a, b) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]
    return [buckets[i] for i in rng.permutation(len(buckets))]


def _must_fail(call):
    with pytest.raises(dp.DpError) as e:
        call()
    assert e.value.status in (dp.DP_ERR_STATE, dp.DP_ERR_INVALID_ARG), e.value


def _snapshot(run):
    torch.cuda.synchronize()
    return run.window(0, run.w.P)


def _same(a, b, where):
    for k in ("w", "m", "v", "p"):
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), f"{where}: {k}"


def _scalars_bits(st):
    return np.array([v for k, v in sorted(st.items()) if k != "bank"], np.float64).view(np.uint64)


CASES = {
    "two_pass_clip": dict(base="gpt2_small", numel=RAGGED, n=3, a=3, max_norm=0.05, scaled_tensors=(4,), steps=2),
    "single_pass": dict(base="tiny", numel=RAGGED, n=3, a=3, steps=2),
}


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("name", sorted(CASES))
def test_random_bucket_schedules_equal_whole(name, seed):
    spec = dict(CASES[name])
    base = workloads.by_name(spec.pop("base"))
    steps = spec.pop("steps")
    w = base.with_(**spec)
    single = w.max_norm == 0.0
    ref_run = DeviceRun(w, single_pass=single)
    try:
        ref_states = ref_run.run(steps)
        ref = _snapshot(ref_run)
    finally:
        ref_run.close()

    rng = np.random.default_rng(1000 + seed)
    grid = _grid(w)
    run = DeviceRun(w, single_pass=single)
    d, pl, s = run.d, run.d.plan, run.stream
    lr, eps, wd = w.lr, w.eps, w.weight_decay
    routes = []
    try:
        for r in range(w.n):
            pl.bind("grad", run.slots[r], r)
        states = []
        for step in range(1, steps + 1):
            for k in range(1, w.a + 1):
                for r in range(w.n):
                    synth.grad_device(w, step, r, k, run.slots[r].data_ptr(), d.scale, s)
                last = k == w.a
                if not last:
                    if rng.random() < 0.3:
                        pl.accumulate_all(first=(k == 1), stream=s)
                        routes.append("whole")
                        continue
                    bs = _partition(rng, grid, w.P)
                    routes.append(f"acc{len(bs)}")
                    for i, (lo, hi) in enumerate(bs):
                        pl.accumulate_all_range(k == 1, lo, hi, stream=s)
                        if i + 1 < len(bs) and rng.random() < 0.5:  # half done: these must refuse
                            _must_fail([lambda: pl.grad_stats(False, w.max_norm, stream=s),
                                        lambda: pl.accumulate_all(k == 1, stream=s),
                                        lambda: pl.accumulate_all_range(k != 1, *bs[i + 1], stream=s),
                                        lambda: pl.accumulate_all_range(k == 1, lo, hi, stream=s),
                                        lambda: pl.accumulate_reduce_range(*bs[i + 1], stream=s)]
                                       [int(rng.integers(0, 5))])
                    continue
                # the last micro-step
                if single:
                    if rng.random() < 0.3:
                        pl.reduce_adam_step(lr, eps, wd, stream=s)
                        routes.append("single-whole")
                    else:
                        bs = _partition(rng, grid, w.P)
                        routes.append(f"single{len(bs)}")
                        for i, (lo, hi) in enumerate(bs):
                            pl.reduce_adam_range(lr, eps, wd, lo, hi, stream=s)
                            if i + 1 < len(bs) and rng.random() < 0.5:
                                _must_fail([lambda: pl.reduce_adam_finish(stream=s),
                                            lambda: pl.reduce_adam_range(2 * lr, eps, wd, *bs[i + 1], stream=s),
                                            lambda: pl.accumulate_all(False, stream=s),
                                            lambda: pl.reduce_adam_step(lr, eps, wd, stream=s)]
                                           [int(rng.integers(0, 4))])
                        pl.reduce_adam_finish(stream=s)
                else:
                    route = int(rng.integers(0, 3))
                    if route == 0:
                        pl.accumulate_reduce(stream=s)
                        routes.append("reduce-whole")
                    elif route == 1:
                        bs = _partition(rng, grid, w.P)
                        routes.append(f"reduce{len(bs)}")
                        for i, (lo, hi) in enumerate(bs):
                            pl.accumulate_reduce_range(lo, hi, stream=s)
                            if i + 1 < len(bs) and rng.random() < 0.5:
                                _must_fail([lambda: pl.grad_stats(False, w.max_norm, stream=s),
                                            lambda: pl.reduce_replicas_range("acc", *bs[i + 1], stream=s),
                                            lambda: pl.accumulate_reduce_range(lo, hi, stream=s)]
                                           [int(rng.integers(0, 3))])
                    else:  # the last micro-step accumulated, then reduced from the accumulators
                        for lo, hi in _partition(rng, grid, w.P):
                            pl.accumulate_all_range(False, lo, hi, stream=s)
                        bs = _partition(rng, grid, w.P)
                        routes.append(f"acc-then-reduce{len(bs)}")
                        for lo, hi in bs:
                            pl.reduce_replicas_range("acc", lo, hi, stream=s)
                    _must_fail(lambda: pl.adam_step(lr, eps, wd, stream=s))  # before the statistics
                    pl.grad_stats(False, w.max_norm, stream=s)
                    pl.adam_step(lr, eps, wd, stream=s)
            st = pl.read_state(stream=s)
            d.scale = st["scale"]
            states.append(st)
        got = _snapshot(run)
    finally:
        run.close()
    log(f"{name} seed {seed}: {' '.join(routes)}")
    _same(got, ref, f"{name} seed {seed}")
    for i, (a, b) in enumerate(zip(states, ref_states), start=1):
        assert np.array_equal(_scalars_bits(a), _scalars_bits(b)), f"{name} seed {seed} step {i} scalars"
