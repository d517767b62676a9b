"""The bucketed replica reduction (dp_accumulate_reduce_range): the last
micro-step reduced bucket by bucket, on a second stream while the producer
writes the next bucket, in backward order or shuffled, with buckets that
split tensors.  It must give the same bits as the whole-range reduction, and
so agree with the oracle; the ordering rules fail loudly.  The same for the
bucketed single pass (dp_reduce_adam_range, then dp_reduce_adam_finish),
whose buckets also update their parameters, against the whole-range single
pass, skipped steps included; and for the earlier micro-steps accumulated
bucket by bucket (dp_accumulate_all_range)."""
import numpy as np
import pytest
import torch

import gradient_reduce_adam_amd as dp
import synth
from gradient_reduce_adam_amd import driver
from synth import workloads

from gpu_common import DeviceRun, assert_scalars_match, assert_state_close, log, oracle_run, ulp_bound

pytestmark = pytest.mark.gpu

RAGGED = (3000, 17, 4096, 5, 70001, 256, 1, 65536, 131075)


def _split_inside(buckets, w):
    """Splits every bucket longer than 2048 elements once more, 256 * k
    elements into the tensor that holds its midpoint."""
    off = [int(x) for x in w.offsets]
    out = []
    for lo, hi in buckets:
        mid = (lo + hi) // 2
        t = max(i for i in range(w.T) if off[i] <= mid)
        cut = off[t] + (mid - off[t]) // 256 * 256
        if hi - lo > 2048 and lo < cut < hi:
            out += [(cut, hi), (lo, cut)]
        else:
            out.append((lo, hi))
    return out


def _bucketed_run(w, steps, buckets, two_streams, single=False, micro=False):
    run = DeviceRun(w, single_pass=single)
    d = run.d
    slots = [torch.empty(w.P, dtype=torch.int16, device="cuda") for _ in range(w.n)]
    addrs = [t.data_ptr() for t in slots]

    def produce(step, k, lo, hi, stream):
        for r in range(w.n):
            synth.grad_device(w, step, r, k, addrs[r] + 2 * lo, d.scale, stream, lo, hi)

    rs = torch.cuda.Stream() if two_streams else None
    try:
        states = [d.step_overlapped(addrs, produce, buckets, reduce_stream=rs, micro_buckets=micro)
                  for _ in range(steps)]
        return run.window(0, w.P), states
    finally:
        run.close()
        del slots


def _whole_run(w, steps, single=False):
    run = DeviceRun(w, single_pass=single)
    try:
        states = run.run(steps)
        return run.window(0, w.P), states
    finally:
        run.close()


def _same(a, b):
    (wa, sa), (wb, sb) = a, b
    assert wa.keys() == wb.keys()
    for k in wa:
        assert np.array_equal(wa[k].view(np.uint8), wb[k].view(np.uint8)), k
    for x, y in zip(sa, sb):
        assert np.array_equal(np.array(list(x.values()), np.float64).view(np.uint64),
                              np.array(list(y.values()), np.float64).view(np.uint64))


CASES = {
    "clip_n3_a2": dict(base="gpt2_small", numel=RAGGED, n=3, a=2, max_norm=0.05, scaled_tensors=(4,), steps=3),
    "partials_dynamic": dict(base="zero3_rank_7b", numel=RAGGED, n=4, a=1, growth_interval=2, steps=4,
                             injections=((2, 1, 1, 70000, float("inf")),)),
    "n1_a3": dict(base="unsharded_7b", numel=RAGGED, n=1, a=3, steps=2),
}


@pytest.mark.parametrize("two_streams", [False, True])
@pytest.mark.parametrize("name", sorted(CASES))
def test_bucketed_reduction_equals_whole_bitwise(name, two_streams):
    spec = dict(CASES[name])
    base = workloads.by_name(spec.pop("base"))
    steps = spec.pop("steps")
    w = base.with_(**spec)
    buckets = _split_inside(driver.backward_buckets(w.numel, 64 << 10), w)
    log(f"buckets {name} two_streams={two_streams}: {len(buckets)} buckets")
    got = _bucketed_run(w, steps, buckets, two_streams)
    _same(got, _whole_run(w, steps))
    if two_streams:  # and the oracle agrees
        ref = oracle_run(w, steps)
        for s, (g, r) in enumerate(zip(got[1], ref.scalars), start=1):
            assert_scalars_match(g, r, where=f"{name} step {s}")
        assert_state_close(got[0], ref.state[(0, w.P)], ulp_bound(w), where=name)


def test_shuffled_buckets_equal_whole_bitwise():
    w = workloads.gpt2_small().with_(numel=RAGGED, n=2, a=2, max_norm=0.05, scaled_tensors=(1,))
    rng = np.random.default_rng(7)
    buckets = _split_inside(driver.backward_buckets(w.numel, 16 << 10), w)
    buckets = [buckets[i] for i in rng.permutation(len(buckets))]
    log(f"shuffled buckets: {buckets}")
    _same(_bucketed_run(w, 2, buckets, True), _whole_run(w, 2))


def test_bucket_ordering_errors():
    w = workloads.gpt2_small().with_(numel=(5000, 3000, 700), n=2, a=1, scaled_tensors=())
    run = DeviceRun(w)
    d, pl, s = run.d, run.d.plan, run.stream
    try:
        for r in range(w.n):
            run.slots[r].zero_()
            pl.bind("grad", run.slots[r], r)
        for lo, hi in ((3, 5000), (0, 4999), (100, 300)):  # ends off the piece grid
            with pytest.raises(dp.DpError) as e:
                pl.accumulate_reduce_range(lo, hi, stream=s)
            assert e.value.status == dp.DP_ERR_INVALID_ARG
        with pytest.raises(dp.DpError) as e:
            pl.accumulate_reduce_range(0, w.P + 1, stream=s)
        assert e.value.status == dp.DP_ERR_RANGE
        pl.accumulate_reduce_range(5000, 8000, stream=s)  # a tensor
        with pytest.raises(dp.DpError) as e:  # overlaps it
            pl.accumulate_reduce_range(5256, 8700, stream=s)
        assert e.value.status == dp.DP_ERR_STATE
        for call in (lambda: pl.grad_stats(False, 0.0, stream=s), lambda: pl.accumulate_all(True, stream=s),
                     lambda: pl.accumulate_reduce(stream=s)):
            with pytest.raises(dp.DpError) as e:  # the reduction is half done
                call()
            assert e.value.status == dp.DP_ERR_STATE and "bucketed" in e.value.message
        pl.accumulate_reduce_range(256, 5000, stream=s)  # 256 elements into tensor 0
        pl.accumulate_reduce_range(8000, 8700, stream=s)
        pl.accumulate_reduce_range(0, 256, stream=s)  # complete now
        pl.grad_stats(False, 0.0, stream=s)
        pl.adam_step(w.lr, w.eps, w.weight_decay, stream=s)
        assert pl.read_state(stream=s)["t"] == 1
    finally:
        run.close()


SINGLE_CASES = {
    # ZeRO-style partials, dynamic scale that grows, an inf that skips step 2
    "partials_dynamic_skip": dict(base="zero3_rank_7b", numel=RAGGED, n=4, a=1, growth_interval=2, steps=4,
                                  injections=((2, 1, 1, 70000, float("inf")),)),
    "n3_a2": dict(base="tiny", numel=RAGGED, n=3, a=2, steps=3),
    "n1_a3": dict(base="unsharded_7b", numel=RAGGED, n=1, a=3, steps=2),
}


@pytest.mark.parametrize("two_streams", [False, True])
@pytest.mark.parametrize("name", sorted(SINGLE_CASES))
def test_bucketed_single_pass_equals_whole_bitwise(name, two_streams):
    spec = dict(SINGLE_CASES[name])
    base = workloads.by_name(spec.pop("base"))
    steps = spec.pop("steps")
    w = base.with_(**spec)
    buckets = _split_inside(driver.backward_buckets(w.numel, 64 << 10), w)
    log(f"single-pass buckets {name} two_streams={two_streams}: {len(buckets)} buckets")
    got = _bucketed_run(w, steps, buckets, two_streams, single=True)
    _same(got, _whole_run(w, steps, single=True))
    if two_streams:
        ref = oracle_run(w, steps)
        for s, (g, r) in enumerate(zip(got[1], ref.scalars), start=1):
            assert_scalars_match(g, r, where=f"{name} step {s}")
        assert_state_close(got[0], ref.state[(0, w.P)], ulp_bound(w), where=name)


def test_shuffled_single_pass_buckets_equal_whole_bitwise():
    w = workloads.tiny().with_(numel=RAGGED, n=2, a=2)
    rng = np.random.default_rng(11)
    buckets = _split_inside(driver.backward_buckets(w.numel, 16 << 10), w)
    buckets = [buckets[i] for i in rng.permutation(len(buckets))]
    _same(_bucketed_run(w, 3, buckets, True, single=True), _whole_run(w, 3, single=True))


def test_single_pass_bucket_ordering_errors():
    w = workloads.tiny().with_(numel=(5000, 3000, 700), n=2, a=1)
    run = DeviceRun(w, single_pass=True)
    pl, s = run.d.plan, run.stream
    lr, eps, wd = w.lr, w.eps, w.weight_decay
    try:
        for r in range(w.n):
            run.slots[r].zero_()
            pl.bind("grad", run.slots[r], r)
        with pytest.raises(dp.DpError) as e:  # nothing done yet
            pl.reduce_adam_finish(stream=s)
        assert e.value.status == dp.DP_ERR_STATE
        pl.reduce_adam_range(lr, eps, wd, 5000, 8000, stream=s)
        with pytest.raises(dp.DpError) as e:  # other hyperparameters in the same step
            pl.reduce_adam_range(2 * lr, eps, wd, 0, 5000, stream=s)
        assert e.value.status == dp.DP_ERR_INVALID_ARG
        with pytest.raises(dp.DpError) as e:  # overlap
            pl.reduce_adam_range(lr, eps, wd, 5256, 8700, stream=s)
        assert e.value.status == dp.DP_ERR_STATE
        with pytest.raises(dp.DpError) as e:  # the other kind of bucket
            pl.accumulate_reduce_range(0, 5000, stream=s)
        assert e.value.status == dp.DP_ERR_STATE
        for call in (lambda: pl.reduce_adam_step(lr, eps, wd, stream=s), lambda: pl.grad_stats(False, 0.0, stream=s),
                     lambda: pl.accumulate_all(True, stream=s), lambda: pl.accumulate_reduce(stream=s)):
            with pytest.raises(dp.DpError) as e:
                call()
            assert e.value.status == dp.DP_ERR_STATE and "single pass" in e.value.message
        with pytest.raises(dp.DpError) as e:  # 3000 + 700 of 8700 elements missing
            pl.reduce_adam_finish(stream=s)
        assert e.value.status == dp.DP_ERR_STATE
        pl.reduce_adam_range(lr, eps, wd, 8000, 8700, stream=s)
        pl.reduce_adam_range(lr, eps, wd, 0, 5000, stream=s)
        pl.reduce_adam_finish(stream=s)
        st = pl.read_state(stream=s)
        assert st["t"] == 1 and st["bank"] == 1
        pl.reduce_adam_step(lr, eps, wd, stream=s)  # a whole-range step works again
        assert pl.read_state(stream=s)["t"] == 2
    finally:
        run.close()


MICRO_CASES = {
    "clip_n3_a2": (CASES["clip_n3_a2"], False),
    "n1_a3": (CASES["n1_a3"], False),
    "single_n3_a2": (SINGLE_CASES["n3_a2"], True),
    "single_n1_a3": (SINGLE_CASES["n1_a3"], True),
}


@pytest.mark.parametrize("two_streams", [False, True])
@pytest.mark.parametrize("name", sorted(MICRO_CASES))
def test_bucketed_micro_steps_equal_whole_bitwise(name, two_streams):
    """Every micro-step accumulated bucket by bucket as the producer writes
    it, the last one reduced (or reduced and applied) bucket by bucket: the
    same bits as the whole-range step; on two streams the producer reuses the
    gradient buffers while earlier buckets are still being added."""
    spec, single = dict(MICRO_CASES[name][0]), MICRO_CASES[name][1]
    base = workloads.by_name(spec.pop("base"))
    steps = spec.pop("steps")
    w = base.with_(**spec)
    buckets = _split_inside(driver.backward_buckets(w.numel, 64 << 10), w)
    log(f"micro-step buckets {name} two_streams={two_streams}: {len(buckets)} buckets")
    got = _bucketed_run(w, steps, buckets, two_streams, single=single, micro=True)
    _same(got, _whole_run(w, steps, single=single))
    if two_streams:
        ref = oracle_run(w, steps)
        for s, (g, r) in enumerate(zip(got[1], ref.scalars), start=1):
            assert_scalars_match(g, r, where=f"{name} step {s}")
        assert_state_close(got[0], ref.state[(0, w.P)], ulp_bound(w), where=name)


def test_shuffled_micro_step_buckets_equal_whole_bitwise():
    w = workloads.gpt2_small().with_(numel=RAGGED, n=2, a=3, max_norm=0.05, scaled_tensors=(1,))
    rng = np.random.default_rng(13)
    buckets = _split_inside(driver.backward_buckets(w.numel, 16 << 10), w)
    buckets = [buckets[i] for i in rng.permutation(len(buckets))]
    _same(_bucketed_run(w, 2, buckets, True, micro=True), _whole_run(w, 2))


def test_micro_step_bucket_ordering_errors():
    w = workloads.gpt2_small().with_(numel=(5000, 3000, 700), n=2, a=3, scaled_tensors=())
    run = DeviceRun(w)
    pl, s = run.d.plan, run.stream
    try:
        for r in range(w.n):
            run.slots[r].zero_()
            pl.bind("grad", run.slots[r], r)
        with pytest.raises(dp.DpError) as e:  # no first micro-step yet
            pl.accumulate_all_range(False, 0, 5000, stream=s)
        assert e.value.status == dp.DP_ERR_STATE
        for lo, hi in ((3, 5000), (0, 4999)):  # ends off the piece grid
            with pytest.raises(dp.DpError) as e:
                pl.accumulate_all_range(True, lo, hi, stream=s)
            assert e.value.status == dp.DP_ERR_INVALID_ARG
        pl.accumulate_all_range(True, 5000, 8000, stream=s)
        with pytest.raises(dp.DpError) as e:  # another first flag in the same micro-step
            pl.accumulate_all_range(False, 0, 5000, stream=s)
        assert e.value.status == dp.DP_ERR_INVALID_ARG
        with pytest.raises(dp.DpError) as e:  # overlap
            pl.accumulate_all_range(True, 5256, 8700, stream=s)
        assert e.value.status == dp.DP_ERR_STATE
        with pytest.raises(dp.DpError) as e:  # the other kinds of bucket
            pl.accumulate_reduce_range(0, 5000, stream=s)
        assert e.value.status == dp.DP_ERR_STATE
        with pytest.raises(dp.DpError) as e:
            pl.reduce_adam_range(w.lr, w.eps, w.weight_decay, 0, 5000, stream=s)
        assert e.value.status == dp.DP_ERR_STATE
        for call in (lambda: pl.accumulate_all(False, stream=s), lambda: pl.accumulate(0, True, stream=s),
                     lambda: pl.accumulate_reduce(stream=s), lambda: pl.grad_stats(False, 0.0, stream=s),
                     lambda: pl.reduce_replicas("acc", stream=s)):
            with pytest.raises(dp.DpError) as e:  # the micro-step is half done
                call()
            assert e.value.status == dp.DP_ERR_STATE and "micro-step" in e.value.message
        pl.accumulate_all_range(True, 0, 5000, stream=s)
        pl.accumulate_all_range(True, 8000, 8700, stream=s)  # complete: micro-step 1
        pl.accumulate_all_range(False, 0, 8700, stream=s)  # micro-step 2 as one bucket
        pl.accumulate_reduce(stream=s)  # micro-step 3 fused with the reduction
        pl.grad_stats(False, 0.0, stream=s)
        pl.adam_step(w.lr, w.eps, w.weight_decay, stream=s)
        assert pl.read_state(stream=s)["t"] == 1
    finally:
        run.close()


def _reduce_replicas_bucketed_run(w, steps, buckets, src):
    """Every micro-step accumulated whole (or, for partials, none), then the
    replica reduction from ACC or from the partials bucket by bucket
    (dp_reduce_replicas_range); statistics and update whole."""
    run = DeviceRun(w)
    d, pl, st = run.d, run.d.plan, run.stream
    try:
        states = []
        for step in range(1, steps + 1):
            last = 1 if w.partials else w.a
            for k in range(1, last + 1):
                for r in range(w.n):
                    synth.grad_device(w, step, r, k, run.slots[r].data_ptr(), d.scale, st)
                    pl.bind("grad", run.slots[r], r)
                if src == "acc":
                    pl.accumulate_all(first=(k == 1), stream=st)
            for lo, hi in buckets:
                pl.reduce_replicas_range(src, lo, hi, stream=st)
            d.finish()
            states.append(d.read_state())
            d.scale = states[-1]["scale"]
        return run.window(0, w.P), states
    finally:
        run.close()


@pytest.mark.parametrize("name,src", [("clip_n3_a2", "acc"), ("n1_a3", "acc"), ("partials_dynamic", "grad")])
def test_bucketed_reduce_replicas_equals_whole_bitwise(name, src):
    """The reduction from the accumulators after every micro-step (or from
    incoming partials) in shuffled buckets that split tensors: the g_bar,
    statistics and state of the fused whole-range step, and the oracle's."""
    spec = dict(CASES[name])
    base = workloads.by_name(spec.pop("base"))
    steps = spec.pop("steps")
    w = base.with_(**spec)
    rng = np.random.default_rng(17)
    buckets = _split_inside(driver.backward_buckets(w.numel, 32 << 10), w)
    buckets = [buckets[i] for i in rng.permutation(len(buckets))]
    log(f"reduce_replicas_range {name} src={src}: {len(buckets)} buckets")
    got = _reduce_replicas_bucketed_run(w, steps, buckets, src)
    _same(got, _whole_run(w, steps))
    ref = oracle_run(w, steps)
    for s, (g, r) in enumerate(zip(got[1], ref.scalars), start=1):
        assert_scalars_match(g, r, where=f"{name} step {s}")
    assert_state_close(got[0], ref.state[(0, w.P)], ulp_bound(w), where=name)


def test_reduce_replicas_bucket_errors():
    w = workloads.gpt2_small().with_(numel=(5000, 3000, 700), n=2, a=2, scaled_tensors=())
    run = DeviceRun(w)
    pl, s = run.d.plan, run.stream
    try:
        for r in range(w.n):
            run.slots[r].zero_()
            pl.bind("grad", run.slots[r], r)
        with pytest.raises(dp.DpError) as e:  # no micro-step accumulated yet
            pl.reduce_replicas_range("acc", 0, 5000, stream=s)
        assert e.value.status == dp.DP_ERR_STATE
        pl.accumulate_all(True, stream=s)
        pl.accumulate_all(False, stream=s)
        pl.reduce_replicas_range("acc", 5000, 8000, stream=s)
        for call in (lambda: pl.reduce_replicas_range("grad", 0, 5000, stream=s),
                     lambda: pl.accumulate_reduce_range(0, 5000, stream=s)):
            with pytest.raises(dp.DpError) as e:  # other sources in the same reduction
                call()
            assert e.value.status == dp.DP_ERR_INVALID_ARG
        with pytest.raises(dp.DpError) as e:  # overlap
            pl.reduce_replicas_range("acc", 5256, 8700, stream=s)
        assert e.value.status == dp.DP_ERR_STATE
        with pytest.raises(dp.DpError) as e:  # the reduction is half done
            pl.reduce_replicas("acc", stream=s)
        assert e.value.status == dp.DP_ERR_STATE and "bucketed" in e.value.message
        pl.reduce_replicas_range("acc", 0, 5000, stream=s)
        pl.reduce_replicas_range("acc", 8000, 8700, stream=s)  # complete
        pl.grad_stats(False, 0.0, stream=s)
        pl.adam_step(w.lr, w.eps, w.weight_decay, stream=s)
        assert pl.read_state(stream=s)["t"] == 1
    finally:
        run.close()


def test_bucketed_micro_steps_on_misaligned_per_tensor_bindings():
    """Three micro-steps of three replicas accumulated bucket by bucket (in a
    shuffled order) into per-tensor accumulators shifted off 16-byte
    alignment, from per-tensor gradients shifted likewise: the table path and
    the per-element path of the ranged call.  The accumulators must equal,
    bit for bit, those of the whole-space call on flat buffers."""
    w = workloads.tiny().with_(numel=RAGGED, n=3, a=3)
    P, T, off = w.P, w.T, [int(x) for x in w.offsets]
    s = torch.cuda.current_stream().cuda_stream
    grads = {}
    for k in range(1, w.a + 1):
        for r in range(w.n):
            g = torch.empty(P, dtype=torch.int16, device="cuda")
            synth.grad_device(w, 1, r, k, g.data_ptr(), 1.0, s)
            grads[(k, r)] = g

    def split(back):  # tensor t at element off[t] + t + 1 of its backing buffer
        return [back[off[t] + t + 1:off[t + 1] + t + 1] for t in range(T)]

    flat_acc = torch.zeros((w.n, P), dtype=torch.float32, device="cuda")
    ref = dp.Plan(w.numel, w.n, w.grad_dtype, w.param_dtype)
    test = dp.Plan(w.numel, w.n, w.grad_dtype, w.param_dtype)
    acc_backs = [torch.full((P + T + 1,), float("nan"), dtype=torch.float32, device="cuda") for _ in range(w.n)]
    try:
        for r in range(w.n):
            ref.bind("acc", flat_acc[r], r)
            test.bind_tensors("acc", split(acc_backs[r]), r)
        buckets = _split_inside(driver.backward_buckets(w.numel, 16 << 10), w)
        rng = np.random.default_rng(19)
        keep = []
        for k in range(1, w.a + 1):
            for r in range(w.n):
                ref.bind("grad", grads[(k, r)], r)
                gb = torch.zeros(P + T + 1, dtype=torch.int16, device="cuda")
                for t, piece in enumerate(split(gb)):
                    piece.copy_(grads[(k, r)][off[t]:off[t + 1]])
                keep.append(gb)
                test.bind_tensors("grad", split(gb), r)
            ref.accumulate_all(first=(k == 1), stream=s)
            for i in rng.permutation(len(buckets)):
                lo, hi = buckets[i]
                test.accumulate_all_range(k == 1, lo, hi, stream=s)
            torch.cuda.synchronize()  # the per-tensor GRAD tables are rewritten for the next micro-step
        for r in range(w.n):
            got = torch.cat(split(acc_backs[r])).view(torch.int32).cpu().numpy()
            want = flat_acc[r].view(torch.int32).cpu().numpy()
            assert np.array_equal(got, want), r
    finally:
        ref.close()
        test.close()
