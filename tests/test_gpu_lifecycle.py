"""The plan's life cycle on the GPU, through the C ABI: a failed allocation of
the state leaves nothing behind and the plan usable for error reporting;
per-tensor pointer tables rebound between launches on a non-default stream
never reach a kernel that was launched with the old ones, a rebinding does
not wait for the device, and launches on two streams read a rebound table
after its upload; and cached range tables can be dropped when the shard
partition changes during a run."""
import time

import numpy as np
import pytest
import torch

import gradient_reduce_adam_amd as dp
import synth
from gradient_reduce_adam_amd import driver
from synth import workloads

from gpu_common import assert_scalars_match, assert_state_close, log, oracle_run, ulp_bound

pytestmark = pytest.mark.gpu


def test_state_allocation_failure_is_clean():
    # 2^46 elements in chunks of 2^26: a small chunk table (2^20 entries), but
    # statistics scratch for 2^38 pieces (several TB), which no GPU holds
    plan = dp.Plan((1 << 46,), 1, "bf16", "bf16", chunk_elems=1 << 26)
    try:
        for attempt in range(2):
            with pytest.raises(dp.DpError) as e:
                plan.state_init(0.9, 0.999)
            assert e.value.status in (dp.DP_ERR_OOM, dp.DP_ERR_HIP), e.value
            log(f"attempt {attempt}: {e.value}")
        with pytest.raises(dp.DpError) as e:  # no state block was kept
            plan.read_state()
        assert e.value.status == dp.DP_ERR_STATE
    finally:
        plan.close()


def test_rebinding_pointer_tables_between_launches():
    """Every micro-step's gradients sit in their own buffers, one pointer per
    tensor, and the GRAD tables are rebound before every launch while the
    previous launch may still run on a non-default stream.  The result must
    be the oracle's."""
    w = workloads.gpt2_small().with_(numel=(1001, 4099, 65536 + 3, 70001), n=2, a=3, max_norm=0.05,
                                     scaled_tensors=(), steps=2)
    P, off, T = w.P, w.offsets, w.T
    dev = "cuda"
    stream = torch.cuda.Stream()
    s = stream.cuda_stream

    def tensors(back):
        return [back[int(off[t]) + t + 1:int(off[t + 1]) + t + 1] for t in range(T)]

    # every (step, micro-step, replica) gradient, generated up front
    grads = {}
    flat = torch.empty(P, dtype=torch.int16, device=dev)
    for st in range(1, w.steps + 1):
        for k in range(1, w.a + 1):
            for r in range(w.n):
                synth.grad_device(w, st, r, k, flat.data_ptr(), 1.0, torch.cuda.current_stream().cuda_stream)
                back = torch.zeros(P + T + 1, dtype=torch.int16, device=dev)
                ts = tensors(back)
                for t in range(T):
                    ts[t].copy_(flat[int(off[t]):int(off[t + 1])])
                grads[(st, k, r)] = (back, ts)
    master = torch.empty(P, dtype=torch.float32, device=dev)
    synth.master_device(w, master.data_ptr(), torch.cuda.current_stream().cuda_stream)
    m = torch.zeros(P, dtype=torch.float32, device=dev)
    v = torch.zeros(P, dtype=torch.float32, device=dev)
    p = master.to(torch.bfloat16)
    acc = torch.zeros((w.n, P), dtype=torch.float32, device=dev)
    gbar = torch.zeros(P, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    plan = dp.Plan(w.numel, w.n, w.grad_dtype, w.param_dtype)
    try:
        plan.bind("master", master)
        plan.bind("exp_avg", m)
        plan.bind("exp_avg_sq", v)
        plan.bind("param", p)
        plan.bind("gbar", gbar)
        for r in range(w.n):
            plan.bind("acc", acc[r], r)
        plan.state_init(w.beta1, w.beta2, stream=s)
        for st in range(1, w.steps + 1):
            for k in range(1, w.a + 1):
                for r in range(w.n):
                    plan.bind_tensors("grad", grads[(st, k, r)][1], r)
                if k < w.a:
                    plan.accumulate_all(first=(k == 1), stream=s)
                else:
                    plan.accumulate_reduce(stream=s)
            plan.grad_stats(False, w.max_norm, stream=s)
            plan.adam_step(w.lr, w.eps, w.weight_decay, stream=s)
        state = plan.read_state(stream=s)
        got = {"w": master.cpu().numpy(), "m": m.cpu().numpy(), "v": v.cpu().numpy(),
               "p": p.view(torch.int16).cpu().numpy().view(np.uint16)}
    finally:
        plan.close()
    ref = oracle_run(w, w.steps)
    assert_scalars_match(state, ref.scalars[-1], where="rebound tables")
    assert_state_close(got, ref.state[(0, P)], ulp_bound(w), where="rebound tables")


def test_shard_ranges_change_over_a_run():
    """The update runs over 3 shard ranges for two steps; the cached range
    tables are dropped and the next two steps run over 5 other ranges.  The
    result is the oracle's: a partition of the range never changes the
    update, and dropped tables are rebuilt on demand."""
    w = workloads.tiny().with_(numel=(3000, 17, 70001, 4096, 131075), n=2, a=2, steps=4)
    P = w.P
    d = driver.DPStep(w.numel, w.n, w.a, w.grad_dtype, w.param_dtype, lr=w.lr, eps=w.eps,
                      weight_decay=w.weight_decay, beta1=w.beta1, beta2=w.beta2)
    s = d.stream.cuda_stream
    d.set_master(lambda ptr: synth.master_device(w, ptr, s))
    slots = [torch.empty(P, dtype=torch.int16, device="cuda") for _ in range(w.n)]

    def produce(step, r, k, scale):
        synth.grad_device(w, step, r, k, slots[r].data_ptr(), scale, s)
        return slots[r].data_ptr()

    try:
        for shards in (driver.even_shards(P, 3), driver.even_shards(P, 5)):
            d.plan.drop_ranges()
            d.shards = shards
            for _ in range(2):
                state = d.step(produce)
        got = {"w": d.master.cpu().numpy(), "m": d.exp_avg.cpu().numpy(), "v": d.exp_avg_sq.cpu().numpy(),
               "p": d.param.view(torch.int16).cpu().numpy().view(np.uint16)}
    finally:
        d.close()
    ref = oracle_run(w, 4)
    assert_scalars_match(state, ref.scalars[-1], where="changing shards")
    assert_state_close(got, ref.state[(0, P)], ulp_bound(w), where="changing shards")


def _busy(stream, products: int = 60):
    """Queues binary32 matrix products of 8192 x 8192 (about 7 ms each) on
    `stream` and returns an event recorded behind them."""
    with torch.cuda.stream(stream):
        a = torch.randn(8192, 8192, device="cuda") * (1.0 / 8192)
        for _ in range(products):
            a = a @ a
        ev = torch.cuda.Event()
        ev.record(stream)
    return ev, a


def test_rebinding_does_not_wait_for_the_gpu():
    """A per-tensor rebinding returns while earlier work still runs on the
    device, and the next launch reads the new pointers."""
    numel = (4099, 70001, 256)
    P, T = sum(numel), len(numel)
    off = np.concatenate([[0], np.cumsum(numel)])
    stream = torch.cuda.Stream()
    s = stream.cuda_stream
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3)
    g = [(torch.randn(P, generator=gen, device="cuda") * 1e-3).to(torch.bfloat16) for _ in range(2)]
    acc = torch.zeros(P, dtype=torch.float32, device="cuda")

    def per_tensor(buf):
        return [buf[int(off[t]):int(off[t + 1])] for t in range(T)]

    plan = dp.Plan(numel, 1, "bf16", "bf16")
    try:
        plan.bind("acc", acc, 0)
        plan.bind_tensors("grad", per_tensor(g[0]), 0)  # the first binding allocates the ring
        plan.accumulate_all(first=True, stream=s)
        torch.cuda.synchronize()
        ev, keep = _busy(stream)
        waits = []
        for i, k in enumerate((1, 0, 1)):  # three rebindings, each followed by a launch behind the busy work
            t = time.perf_counter()
            plan.bind_tensors("grad", per_tensor(g[k]), 0)
            waits.append(time.perf_counter() - t)
            plan.accumulate_all(first=(i == 0), stream=s)
        still_busy = not ev.query()
        torch.cuda.synchronize()
        log(f"rebinding took {[f'{x * 1e3:.3f} ms' for x in waits]}; GPU still busy after them: {still_busy}")
        assert still_busy, "the busy work finished before the rebindings: the check says nothing"
        assert max(waits) < 0.05
        # g[1] as the first micro-step, then g[0] and g[1] added, in binary32
        want = g[1].float() + g[0].float() + g[1].float()
        assert torch.equal(acc.view(torch.int32), want.view(torch.int32))
        del keep
    finally:
        plan.close()


def test_rebound_tables_read_from_two_streams():
    """Micro-steps in buckets, the even buckets on one stream and the odd on
    another, with the GRAD table rebound before every micro-step: the first
    launch after a rebinding uploads the table on its stream and the other
    stream waits for that upload.  Six rebindings wrap the ring of four slots.
    The accumulators equal the binary32 sums bit for bit."""
    numel = (3000, 17, 70001, 4096, 65536 + 256)
    P, T = sum(numel), len(numel)
    off = np.concatenate([[0], np.cumsum(numel)])
    micro = 6
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    g = [(torch.randn(P, generator=gen, device="cuda") * 1e-3).to(torch.bfloat16) for _ in range(micro)]
    acc = torch.zeros(P, dtype=torch.float32, device="cuda")
    buckets = driver.backward_buckets(numel, 16 << 10)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    plan = dp.Plan(numel, 1, "bf16", "bf16")
    try:
        plan.bind("acc", acc, 0)
        for k in range(micro):
            plan.bind_tensors("grad", [g[k][int(off[t]):int(off[t + 1])] for t in range(T)], 0)
            for i, (lo, hi) in enumerate(buckets):
                plan.accumulate_all_range(k == 0, lo, hi, stream=streams[i % 2].cuda_stream)
        torch.cuda.synchronize()
    finally:
        plan.close()
    want = g[0].float()
    for k in range(1, micro):
        want = want + g[k].float()
    log(f"{len(buckets)} buckets on two streams, {micro} rebound micro-steps")
    assert torch.equal(acc.view(torch.int32), want.view(torch.int32))


def _bind_every_role_per_tensor(d, w):
    off = [int(x) for x in w.offsets[:-1]]

    def per(t):
        return [t.data_ptr() + o * t.element_size() for o in off]

    for b, (w_, m_, v_) in enumerate(d.banks):
        for role, t in (("master", w_), ("exp_avg", m_), ("exp_avg_sq", v_)):
            d.plan.bind_tensors(role, per(t), b)
    d.plan.bind_tensors("param", per(d.param))
    for r, t in enumerate(d.acc):
        d.plan.bind_tensors("acc", per(t), r)
    if d.gbar is not None and not (w.n == 1 and not w.partials):
        d.plan.bind_tensors("gbar", per(d.gbar))


CALLS_ON_STREAMS = {
    0: dict(numel=(3000, 0, 17, 70001, 4096, 257), n=3, a=3, max_norm=0.05, scaled_tensors=(3,), single=False,
            shards=[(0, 40000), (40000, 77371)]),
    1: dict(numel=(65536, 5, 12289), n=4, a=4, max_norm=0.0, scaled_tensors=(), single=True, shards=None),
    2: dict(numel=(100, 30000, 1, 30000), n=16, a=2, max_norm=1.0, scaled_tensors=(1,), single=False, shards=None,
            scaler="dynamic", init_scale=1024.0, growth_interval=2, injections=((2, 5, 2, 30050, float("inf")),)),
}


@pytest.mark.parametrize("case", sorted(CALLS_ON_STREAMS))
def test_calls_on_random_streams_with_per_tensor_tables(case):
    """Every call of a step on a seeded random one of three streams, the data
    dependencies between calls ordered by the caller's events, every role
    bound per tensor and the gradients rebound per tensor before every
    micro-step across two buffers per replica (so table uploads happen on one
    stream and are read on others, and ring slots are reused while other
    streams hold them): the same bits as the flat run on one stream."""
    spec = dict(CALLS_ON_STREAMS[case])
    single, shards = spec.pop("single"), spec.pop("shards")
    w = workloads.gpt2_small().with_(steps=3, **spec)
    rng = np.random.default_rng(900 + case)
    log(f"calls on streams {case}: P={w.P} T={w.T} n={w.n} a={w.a} single={single} shards={shards}")

    def make():
        return driver.DPStep(w.numel, w.n, w.a, w.grad_dtype, w.param_dtype, lr=w.lr, eps=w.eps,
                             weight_decay=w.weight_decay, beta1=w.beta1, beta2=w.beta2, max_norm=w.max_norm,
                             scaler=w.scaler, init_scale=w.init_scale, backoff=w.backoff, growth=w.growth,
                             growth_interval=w.growth_interval, shards=shards, single_pass=single)

    def window(d):
        torch.cuda.synchronize()
        w_, m_, v_ = d.state_tensors()
        return [x.view(torch.uint8).cpu().numpy() for x in (w_, m_, v_, d.param)]

    slots = [torch.empty(w.P, dtype=torch.int16, device="cuda") for _ in range(w.n)]
    d = make()
    d.set_master(lambda ptr: synth.master_device(w, ptr, d.stream.cuda_stream))

    def produce(step, r, k, scale):
        synth.grad_device(w, step, r, k, slots[r].data_ptr(), scale, d.stream.cuda_stream)
        return slots[r].data_ptr()

    try:
        ref_states = [d.step(produce) for _ in range(w.steps)]
        ref = window(d)
    finally:
        d.close()

    streams = [torch.cuda.Stream() for _ in range(3)]
    off = [int(x) for x in w.offsets[:-1]]
    bufs = [[torch.empty(w.P, dtype=torch.int16, device="cuda") for _ in range(2)] for _ in range(w.n)]
    d = make()
    d.set_master(lambda ptr: synth.master_device(w, ptr, d.stream.cuda_stream))
    _bind_every_role_per_tensor(d, w)
    prev = torch.cuda.Event()
    prev.record(d.stream)

    def on_random_stream():
        s = streams[int(rng.integers(0, 3))]
        s.wait_event(prev)
        return s

    def done(s):
        ev = torch.cuda.Event()
        ev.record(s)
        return ev

    states = []
    try:
        for step in range(1, w.steps + 1):
            for k in range(1, w.a + 1):
                s = on_random_stream()
                for r in range(w.n):
                    b = bufs[r][k & 1]
                    synth.grad_device(w, step, r, k, b.data_ptr(), d.scale, s.cuda_stream)
                    d.plan.bind_tensors("grad", [b.data_ptr() + 2 * o for o in off], r)
                if k < w.a:
                    d.plan.accumulate_all(first=(k == 1), stream=s.cuda_stream)
                elif single:
                    d.plan.reduce_adam_step(w.lr, w.eps, w.weight_decay, stream=s.cuda_stream)
                else:
                    d.plan.accumulate_reduce(stream=s.cuda_stream)
                prev = done(s)
            if not single:
                s = on_random_stream()
                d.plan.grad_stats(scan=False, max_norm=w.max_norm, stream=s.cuda_stream)
                prev = done(s)
                for b_, e_ in (shards or [(0, w.P)]):
                    s = on_random_stream()
                    d.plan.adam_step(w.lr, w.eps, w.weight_decay, b_, e_, stream=s.cuda_stream)
                    prev = done(s)
            d.stream.wait_event(prev)
            st = d.read_state()
            d.scale = st["scale"]
            states.append(st)
            prev = done(d.stream)
        got = window(d)
    finally:
        d.close()
    for a_, b_, k in zip(got, ref, ("w", "m", "v", "p")):
        assert np.array_equal(a_, b_), k
    for x, y in zip(states, ref_states):
        assert np.array_equal(np.array(list(x.values()), np.float64).view(np.uint64),
                              np.array(list(y.values()), np.float64).view(np.uint64))
