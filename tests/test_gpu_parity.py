"""GPU parity: the HIP library, called through the C ABI, against the CPU
oracle on the same seeded inputs, element by element, at sizes the oracle
finishes in seconds (several chunks per tensor and ragged tails)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import workloads
from gradient_reduce_adam_amd import driver
import gradient_reduce_adam_amd as dp

from gpu_common import (DeviceRun, assert_scalars_match, assert_state_close, log, oracle_run, ulps32, ulp_bound)

pytestmark = pytest.mark.gpu


# ----------------------------------------------------------------------------
# the input generator's device twin
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_generator_device_twin_bit_identical(dtype):
    log(f"generator twin {dtype}")
    for (seed, start, count, c) in [(1, 0, 1 << 20, synth.scale_constant(1e-3)),
                                    (5, (1 << 32) - 1000, 300000, synth.scale_constant(1e-4, 1.0, 1024.0)),
                                    (3, 12345, 77777, synth.scale_constant(1e-4, 1.0, 65536.0)),
                                    (2, 7, 5000, np.float32(1e31))]:
        key = synth.stream_key(seed, synth.ROLE_GRAD, 3, 2, 1)
        host = synth.host_normal(key, start, count, c, dtype, threads=4)
        tdt = torch.float32 if dtype == "f32" else torch.int16
        dev = torch.empty(count, dtype=tdt, device="cuda")
        synth.device_normal(key, start, count, c, dtype, dev.data_ptr(), torch.cuda.current_stream().cuda_stream)
        got = dev.cpu().numpy()
        assert got.tobytes() == host.tobytes()


def test_generator_all_replicas_launch_equals_per_replica():
    """The one-launch generator of every replica's gradient (used by the
    synthetic backward pass) writes the same values as the per-replica one,
    injected non-finite values included."""
    w = workloads.gpt2_small().with_(numel=(3000, 17, 4096, 70001), n=5, a=2, scaled_tensors=(1, 3),
                                     injections=((1, 2, 2, 4000, float("inf")),))
    s = torch.cuda.current_stream().cuda_stream
    multi = torch.zeros((w.n, w.P), dtype=torch.int16, device="cuda")
    single = torch.zeros((w.n, w.P), dtype=torch.int16, device="cuda")
    lo, hi = 2000, w.P - 5
    synth.grads_device_replicas(w, 1, 2, [multi[r].data_ptr() for r in range(w.n)], 4.0, s, lo, hi)
    for r in range(w.n):
        synth.grad_device(w, 1, r, 2, single[r].data_ptr() + 2 * lo, 4.0, s, lo, hi)
    assert torch.equal(multi, single)


# ----------------------------------------------------------------------------
# accumulation and reduction are bit-exact
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("gdt,n,a,chunk", [("bf16", 3, 3, 256), ("f16", 4, 2, 0), ("bf16", 1, 5, 512)])
def test_accumulators_and_gbar_bit_exact(gdt, n, a, chunk):
    w = workloads.gpt2_small().with_(numel=(3000, 17, 4096, 5, 70001, 256, 1, 65536), n=n, a=a, grad_dtype=gdt,
                                     param_dtype=gdt, scaled_tensors=(2,), steps=1)
    log(f"accumulate/reduce {gdt} n={n} a={a} chunk={chunk} P={w.P}")
    ref_gbar = oracle_run(w, 1, keep_gbar=(1,)).gbar[1][(0, w.P)]
    # per-replica calls: every accumulator, then g_bar
    run = DeviceRun(w, chunk_elems=chunk, fused=False)
    try:
        run.d.issue_gradients(run.produce, 1)
        torch.cuda.synchronize()
        for r in range(n):
            ref = np.empty(w.P, np.float32)
            for k in range(1, a + 1):
                oracle.accumulate(ref, synth.grad_host(w, 1, r, k, 0, w.P, 1.0), gdt, first=(k == 1))
            got = run.d.acc[r].cpu().numpy()
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"acc[{r}]"
        assert np.array_equal(run.d.gbar.cpu().numpy().view(np.uint32), ref_gbar.view(np.uint32))
    finally:
        run.close()
    # all replicas per launch, the last micro-step fused with the reduction:
    # the accumulators hold micro-steps 1 .. a-1, g_bar the same bits
    run = DeviceRun(w, chunk_elems=chunk, fused=True)
    try:
        run.d.issue_gradients(run.produce, 1)
        torch.cuda.synchronize()
        if n > 1:
            for r in range(n):
                ref = np.empty(w.P, np.float32)
                for k in range(1, a):
                    oracle.accumulate(ref, synth.grad_host(w, 1, r, k, 0, w.P, 1.0), gdt, first=(k == 1))
                if a > 1:
                    got = run.d.acc[r].cpu().numpy()
                    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"fused acc[{r}]"
        assert np.array_equal(run.d.gbar.cpu().numpy().view(np.uint32), ref_gbar.view(np.uint32))
    finally:
        run.close()


def test_partials_reduction_bit_exact():
    w = workloads.zero3_rank_7b().with_(numel=(200003,), injections=())
    log(f"partials reduce P={w.P}")
    run = DeviceRun(w)
    try:
        run.d.issue_gradients(run.produce, 1)
        ref = oracle_run(w, 1, keep_gbar=(1,)).gbar[1][(0, w.P)]
        torch.cuda.synchronize()
        assert np.array_equal(run.d.gbar.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    finally:
        run.close()


# ----------------------------------------------------------------------------
# whole runs, every element
# ----------------------------------------------------------------------------
def _full_parity(w, steps, shards=None, chunk=0, label="", single_pass=False):
    log(f"full parity {label or w.name}: P={w.P} T={w.T} n={w.n} a={w.a} {w.grad_dtype}/{w.param_dtype} "
        f"clip={w.max_norm} scaler={w.scaler} steps={steps} shards={0 if shards is None else len(shards)} "
        f"single_pass={single_pass}")
    run = DeviceRun(w, shards=shards, chunk_elems=chunk, single_pass=single_pass)
    try:
        gpu_states = run.run(steps)
        got = run.window(0, w.P)
    finally:
        run.close()
    ref = oracle_run(w, steps)
    for s, (g, r) in enumerate(zip(gpu_states, ref.scalars), start=1):
        assert_scalars_match(g, r, where=f"step {s}")
    rep = assert_state_close(got, ref.state[(0, w.P)], ulp_bound(w), where=label)
    log(f"  max ulp: {rep}")
    return got, ref, gpu_states


def test_tiny_workload_ten_steps():
    """The tiny workload exactly: 2^20 params, n=4, a=2, fp16, 10 steps."""
    w = workloads.tiny()
    _, ref, _ = _full_parity(w, w.steps)
    assert ref.scalars[-1]["t"] == 10


def test_long_run_grows_the_scale_at_its_interval():
    """2003 steps of the tiny workload's shape (65539 params) under a dynamic
    loss scale with its full growth interval of 2000 clean steps: the scale
    doubles once, at step 2000, and after every step the scalars, and at the
    end master, m and v, equal the oracle's bit for bit."""
    w = workloads.tiny().with_(numel=(65539,), scaler="dynamic", init_scale=1024.0, growth_interval=2000,
                               steps=2003)
    _, ref, states = _full_parity(w, w.steps)
    scales = [s["scale"] for s in states]
    assert scales[1998] == 1024.0 and scales[1999] == 2048.0 and scales[-1] == 2048.0
    assert ref.scalars[-1]["t"] == 2003


RAGGED = (3000, 17, 4096, 5, 70001, 256, 1, 65536, 131075)

VARIANTS = {
    # bf16, clip active, odd replica count, small chunks: many chunks and tails
    "bf16_clip_n3": dict(base="gpt2_small", numel=RAGGED, n=3, a=3, max_norm=0.05, scaled_tensors=(4,), chunk=256,
                         steps=6),
    # fp16 under a static loss scale with clipping, n = 5
    "f16_static_n5": dict(base="tp_column_slice", numel=RAGGED, n=5, a=2, max_norm=0.02, steps=4),
    # dynamic scale, partials, non-finite values on several steps, growth
    "dynamic_partials": dict(base="zero3_rank_7b", numel=RAGGED, n=4, a=1, growth_interval=2, steps=8,
                             injections=((2, 1, 1, 5, float("nan")), (4, 0, 1, 7000, float("inf")),
                                         (4, 2, 1, 7000, float("-inf")), (6, 3, 1, sum(RAGGED) - 1,
                                                                          float("-inf")))),
    # one replica: the last micro-step's accumulation also writes the statistics
    "n1_fused_stats": dict(base="unsharded_7b", numel=RAGGED, n=1, a=4, max_norm=0.02, steps=5),
    # the most replicas the library takes
    "n16": dict(base="tiny", numel=(65536 * 3 + 11,), n=16, a=1, steps=3),
    "f16_partials_n2": dict(base="zero3_rank_7b", numel=(100000, 3), n=2, a=1, grad_dtype="f16",
                            param_dtype="f16", init_scale=1024.0, injections=(), steps=3),
    # more chunks than one fold group: the statistics fold in two levels
    "two_level_fold": dict(base="gpt2_small", numel=(3000011, 1999999, 5), n=2, a=2, max_norm=0.5,
                           scaled_tensors=(1,), chunk=256, steps=3),
    # parameter dtype different from the gradient dtype
    "bf16_grad_f16_param": dict(base="tiny", numel=RAGGED, n=2, a=2, grad_dtype="bf16", param_dtype="f16",
                                steps=3),
    # 3000 tensors of 0 to 700 elements: most shorter than one piece, every
    # tensor end a ragged tail, a chunk table of thousands of entries
    "many_tiny_tensors": dict(base="gpt2_small", numel=tuple(int(x) for x in np.random.default_rng(11).integers(
        0, 701, 3000)), n=3, a=2, max_norm=0.05, scaled_tensors=(7, 2999), steps=3),
    # the largest chunk size: every tensor here is one chunk of up to 2^18 pieces
    "max_chunk": dict(base="gpt2_small", numel=RAGGED, n=2, a=3, max_norm=0.05, scaled_tensors=(1,),
                      chunk=1 << 26, steps=3),
    # degenerate hyperparameters: lr = 0 and no decay leave w unchanged while
    # m and v move; betas of 0 make m = g and v = g^2 with no bias correction;
    # eps = 1 dominates the denominator
    "lr0_wd0": dict(base="tiny", numel=RAGGED, n=2, a=2, lr=0.0, weight_decay=0.0, steps=3),
    "betas0_eps1": dict(base="tiny", numel=RAGGED, n=3, a=1, beta1=0.0, beta2=0.0, eps=1.0, steps=3),
    # all-zero gradients (signed zeros from the generator) under clipping and a
    # growing dynamic scale: norm 0, clip factor 1, the update only decays w
    "zero_grads": dict(base="gpt2_small", numel=RAGGED, n=2, a=2, grad_sigma=0.0, max_norm=1.0, scaled_tensors=(),
                       scaler="dynamic", init_scale=4.0, growth_interval=2, steps=4),
    # finite bf16 gradients whose binary32 sums overflow: step 1 is skipped on
    # an inf the accumulation created; at half the scale the next steps apply,
    # and the second moment rounds to inf in binary32
    "overflow_in_accumulation": dict(base="gpt2_small", numel=RAGGED, n=2, a=4, grad_sigma=5e37, max_norm=0.0,
                                     scaled_tensors=(), scaler="dynamic", init_scale=1.0, growth_interval=2,
                                     steps=3),
}


@pytest.mark.parametrize("name", sorted(VARIANTS))
def test_variant_full_parity(name):
    spec = dict(VARIANTS[name])
    base = workloads.by_name(spec.pop("base"))
    chunk = spec.pop("chunk", 0)
    steps = spec.pop("steps")
    w = base.with_(**spec)
    _full_parity(w, steps, chunk=chunk, label=name)


@pytest.mark.parametrize("name", ["bf16_clip_n3", "f16_static_n5", "n1_fused_stats", "dynamic_partials"])
def test_per_replica_sequence_equals_fused_bitwise(name):
    """dp_accumulate per (micro-step, replica) + dp_reduce_replicas and
    dp_accumulate_all + dp_accumulate_reduce give the same bits."""
    spec = dict(VARIANTS[name])
    base = workloads.by_name(spec.pop("base"))
    chunk = spec.pop("chunk", 0)
    steps = min(spec.pop("steps"), 4)
    w = base.with_(**spec)
    log(f"per-replica vs fused {name}")
    outs = []
    for fused in (False, True):
        run = DeviceRun(w, chunk_elems=chunk, fused=fused)
        try:
            st = run.run(steps)
            outs.append((run.window(0, w.P), st))
        finally:
            run.close()
    (a, sa), (b, sb) = outs
    for k in ("w", "m", "v", "p", "gbar"):
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k
    for x, y in zip(sa, sb):  # same bits, NaN statistics of skipped steps included
        assert np.array_equal(np.array(list(x.values()), np.float64).view(np.uint64),
                              np.array(list(y.values()), np.float64).view(np.uint64))


# ----------------------------------------------------------------------------
# the single pass (reduce + statistics + update in one read of the state,
# committed after the skip decision) against the oracle and against the
# two-pass sequence, bit for bit
# ----------------------------------------------------------------------------
SINGLE_PASS = {
    # accumulators + last micro-step, fp16, four replicas: the tiny workload's shape, ragged
    "acc_f16_n4": dict(base="tiny", numel=RAGGED, n=4, a=3, steps=4),
    # incoming partials under a dynamic scale: skipped steps (NaN, +inf and -inf), growth
    "dynamic_partials": dict(VARIANTS["dynamic_partials"]),
    # one replica, four micro-steps, bf16, small chunks
    "n1_bf16": dict(base="unsharded_7b", numel=RAGGED, n=1, a=4, chunk=256, steps=4),
    # sixteen single-micro-step replicas
    "n16": dict(VARIANTS["n16"]),
    "bf16_grad_f16_param": dict(VARIANTS["bf16_grad_f16_param"]),
    "lr0_wd0": dict(VARIANTS["lr0_wd0"]),
    "betas0_eps1": dict(VARIANTS["betas0_eps1"]),
    "overflow_in_accumulation": dict(VARIANTS["overflow_in_accumulation"]),
}


def _spec(table, name):
    spec = dict(table[name])
    base = workloads.by_name(spec.pop("base"))
    chunk = spec.pop("chunk", 0)
    steps = spec.pop("steps")
    return base.with_(**spec), chunk, steps


@pytest.mark.parametrize("name", sorted(SINGLE_PASS))
def test_single_pass_full_parity(name):
    w, chunk, steps = _spec(SINGLE_PASS, name)
    _full_parity(w, steps, chunk=chunk, label="single pass " + name, single_pass=True)


@pytest.mark.parametrize("name", sorted(SINGLE_PASS))
def test_single_pass_equals_two_pass_bitwise(name):
    w, chunk, steps = _spec(SINGLE_PASS, name)
    log(f"single pass vs two passes {name}")
    outs = []
    for single in (False, True):
        run = DeviceRun(w, chunk_elems=chunk, single_pass=single)
        try:
            st = run.run(steps)
            outs.append((run.window(0, w.P), st))
        finally:
            run.close()
    (a, sa), (b, sb) = outs
    for k in ("w", "m", "v", "p"):
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k
    for x, y in zip(sa, sb):  # every scalar but the bank index, bit for bit
        keys = [k for k in x if k != "bank"]
        assert np.array_equal(np.array([x[k] for k in keys], np.float64).view(np.uint64),
                              np.array([y[k] for k in keys], np.float64).view(np.uint64))
    # the banks alternate with the applied steps only
    applied = sum(1 for s in sb if not s["found_inf"])
    assert sb[-1]["bank"] == applied % 2 and sa[-1]["bank"] == 0


def test_single_pass_skip_leaves_state_and_params_unchanged():
    """A non-finite g_bar discards the speculative update: the current bank,
    the parameters and every scalar but iter and the scale stay as they were."""
    w = workloads.zero3_rank_7b().with_(numel=(70001, 3000), n=3, injections=((2, 1, 1, 4321, float("inf")),))
    run = DeviceRun(w, single_pass=True)
    try:
        s1 = run.step()
        before = run.window(0, w.P)
        s2 = run.step()
        after = run.window(0, w.P)
        assert s1["found_inf"] == 0 and s2["found_inf"] == 1
        assert s2["bank"] == s1["bank"] == 1 and s2["t"] == s1["t"] == 1 and s2["iter"] == 2
        assert s2["scale"] == s1["scale"] * w.backoff
        for k in ("w", "m", "v", "p"):
            assert np.array_equal(before[k].view(np.uint8), after[k].view(np.uint8)), k
        s3 = run.step()
        assert s3["found_inf"] == 0 and s3["bank"] == 0 and s3["t"] == 2
    finally:
        run.close()


@pytest.mark.parametrize("single", [False, True])
def test_spread_layout_equals_packed_bitwise(single):
    """Where the arrays sit in HBM changes nothing but speed."""
    w = workloads.tiny().with_(numel=RAGGED, n=3, a=2, steps=3)
    outs = []
    for layout in ("packed", "spread"):
        run = DeviceRun(w, single_pass=single, layout=layout)
        try:
            assert run.d.layout == layout
            st = run.run(3)
            outs.append((run.window(0, w.P), st))
        finally:
            run.close()
    (a, sa), (b, sb) = outs
    for k in a:
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k
    assert [x["t"] for x in sa] == [x["t"] for x in sb]


def test_sharded_update_equals_unsharded_bitwise():
    """Sharding changes the layout, not the update: eight uneven ranges give
    the same bits as one call on the whole range."""
    w = workloads.gpt2_small().with_(numel=RAGGED, n=2, a=2, max_norm=0.05, scaled_tensors=(1,), steps=3)
    P = w.P
    shards = [(0, 1), (1, 3001), (3001, 3020), (3020, 50000), (50000, 50000), (50000, 150000), (150000, P - 1),
              (P - 1, P)]
    got_sh, ref, _ = _full_parity(w, 3, shards=shards, label="sharded")
    run = DeviceRun(w)
    try:
        run.run(3)
        got_full = run.window(0, P)
    finally:
        run.close()
    for k in ("w", "m", "v", "p"):
        assert np.array_equal(got_sh[k], got_full[k]), k


def _bind_per_tensor(run, w):
    """Binds every role of the run's plan through per-tensor pointer tables
    into the same memory it holds, so the calls run on table pieces."""
    d = run.d
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


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_sharded_update_on_per_tensor_bindings(seed):
    """With per-tensor bindings a shard's update runs on the pieces of the
    whole chunk table that overlap it, clipped to the shard.  Seeded cuts
    inside pieces, on tensor starts and one element past them, plus an empty
    shard, give the bits of one unsharded call on flat bindings, and the
    oracle's result."""
    w = workloads.gpt2_small().with_(numel=RAGGED, n=2, a=2, max_norm=0.05, scaled_tensors=(1,), steps=3)
    P = w.P
    rng = np.random.default_rng(seed)
    cuts = sorted({0, P, int(w.offsets[3]), int(w.offsets[5]) + 1, int(w.offsets[7]) - 3} |
                  {int(x) for x in rng.integers(1, P, 9)})
    shards = list(zip(cuts[:-1], cuts[1:])) + [(cuts[2], cuts[2])]
    rng.shuffle(shards)
    log(f"per-tensor shards, seed {seed}: {sorted(shards)}")
    run = DeviceRun(w, shards=shards)
    try:
        _bind_per_tensor(run, w)
        states = run.run(3)
        got = run.window(0, P)
    finally:
        run.close()
    run = DeviceRun(w)
    try:
        whole = run.run(3)
        got_full = run.window(0, P)
    finally:
        run.close()
    for k in ("w", "m", "v", "p"):
        assert np.array_equal(got[k].view(np.uint8), got_full[k].view(np.uint8)), k
    assert [x["t"] for x in states] == [x["t"] for x in whole]
    ref = oracle_run(w, 3)
    for s_, (g, r) in enumerate(zip(states, ref.scalars), start=1):
        assert_scalars_match(g, r, where=f"step {s_}")
    assert_state_close(got, ref.state[(0, P)], ulp_bound(w), where="per-tensor shards")


def test_bitwise_reproducible():
    w = workloads.gpt2_small().with_(numel=RAGGED, n=8, a=2, max_norm=0.05, scaled_tensors=(3,), steps=2)
    outs = []
    for _ in range(2):
        run = DeviceRun(w)
        try:
            st = run.run(2)
            outs.append((run.window(0, w.P), st))
        finally:
            run.close()
    (a, sa), (b, sb) = outs
    for k in a:
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k
    assert [s["norm"] for s in sa] == [s["norm"] for s in sb]


# ----------------------------------------------------------------------------
# unaligned memory: per-tensor pointers off the 16-byte grid take the
# scalar path
# ----------------------------------------------------------------------------
def test_misaligned_tensor_bindings():
    w = workloads.gpt2_small().with_(numel=(1001, 4099, 65536 + 3), n=2, a=2, max_norm=0.05, scaled_tensors=(),
                                     steps=2)
    log("misaligned bindings")
    P, off = w.P, w.offsets
    plan = dp.Plan(w.numel, w.n, w.grad_dtype, w.param_dtype, 256)
    dev = "cuda"
    # one backing buffer per role, every tensor shifted by one element
    def f32_tensors():
        back = torch.zeros(P + 2 * w.T, dtype=torch.float32, device=dev)
        return back, [back[int(off[t]) + 2 * t + 1:int(off[t + 1]) + 2 * t + 1] for t in range(w.T)]

    master_b, master_t = f32_tensors()
    m_b, m_t = f32_tensors()
    v_b, v_t = f32_tensors()
    gbar_b, gbar_t = f32_tensors()
    acc = [f32_tensors() for _ in range(w.n)]
    p_back = torch.zeros(P + 2 * w.T, dtype=torch.bfloat16, device=dev)
    p_t = [p_back[int(off[t]) + 2 * t + 1:int(off[t + 1]) + 2 * t + 1] for t in range(w.T)]
    g_back = torch.zeros(P + 2 * w.T, dtype=torch.int16, device=dev)
    g_t = [g_back[int(off[t]) + 2 * t + 1:int(off[t + 1]) + 2 * t + 1] for t in range(w.T)]
    g_flat = torch.empty(P, dtype=torch.int16, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    try:
        plan.bind_tensors("master", master_t)
        plan.bind_tensors("exp_avg", m_t)
        plan.bind_tensors("exp_avg_sq", v_t)
        plan.bind_tensors("gbar", gbar_t)
        plan.bind_tensors("param", p_t)
        for r in range(w.n):
            plan.bind_tensors("acc", acc[r][1], r)
            plan.bind_tensors("grad", g_t, r)
        plan.state_init(w.beta1, w.beta2, stream=stream)
        mflat = torch.empty(P, dtype=torch.float32, device=dev)
        synth.master_device(w, mflat.data_ptr(), stream)
        for t in range(w.T):
            master_t[t].copy_(mflat[int(off[t]):int(off[t + 1])])
            p_t[t].copy_(master_t[t].to(torch.bfloat16))
        for s in (1, 2):
            for k in range(1, w.a + 1):
                for r in range(w.n):
                    synth.grad_device(w, s, r, k, g_flat.data_ptr(), 1.0, stream)
                    for t in range(w.T):
                        g_t[t].copy_(g_flat[int(off[t]):int(off[t + 1])])
                    plan.accumulate(r, first=(k == 1), stream=stream)
            plan.reduce_replicas("acc", stream=stream)
            plan.grad_stats(False, w.max_norm, stream=stream)
            plan.adam_step(w.lr, w.eps, w.weight_decay, stream=stream)
        st = plan.read_state(stream=stream)
        got = {"w": torch.cat(master_t).cpu().numpy(), "m": torch.cat(m_t).cpu().numpy(),
               "v": torch.cat(v_t).cpu().numpy(),
               "p": torch.cat(p_t).view(torch.int16).cpu().numpy().view(np.uint16)}
    finally:
        plan.close()
    ref = oracle_run(w, 2)
    assert_scalars_match(st, ref.scalars[-1])
    assert_state_close(got, ref.state[(0, P)], ulp_bound(w), where="misaligned")


# ----------------------------------------------------------------------------
# low-precision emission: round to nearest even on every binary32 pattern
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("pdt", ["bf16", "f16"])
def test_param_emission_rne_all_binary32_patterns(pdt):
    """With a zero gradient and lr = 0 the update leaves every master value as
    it is, so the emitted parameter is the round-to-nearest-even image of each
    binary32 pattern; 2^32 patterns, checked against torch's conversion."""
    P = 1 << 32
    log(f"emission sweep {pdt}")
    plan = dp.Plan((P,), 1, "bf16", pdt)
    dev = "cuda"
    tdt = torch.bfloat16 if pdt == "bf16" else torch.float16
    piece = 1 << 28

    def patterns(i):  # binary32 bit patterns [i * piece - 2^31, (i + 1) * piece - 2^31)
        lo = i * piece - (1 << 31)
        return torch.arange(lo, lo + piece, dtype=torch.int64, device=dev).to(torch.int32)

    try:
        w = torch.empty(P, dtype=torch.float32, device=dev)
        for i in range(P // piece):
            w[i * piece:(i + 1) * piece] = patterns(i).view(torch.float32)
        z = torch.empty(P, dtype=torch.float32, device=dev)
        v = torch.empty(P, dtype=torch.float32, device=dev)
        p = torch.empty(P, dtype=tdt, device=dev)
        g = torch.empty(P, dtype=torch.int16, device=dev)
        for t in (z, v, p, g):  # torch's elementwise launches stay below 2^31 elements
            for i in range(P // piece):
                t[i * piece:(i + 1) * piece].zero_()
        s = torch.cuda.current_stream().cuda_stream
        plan.bind("master", w)
        plan.bind("exp_avg", z)
        plan.bind("exp_avg_sq", v)
        plan.bind("param", p)
        plan.bind("acc", z)
        plan.bind("grad", g)
        plan.state_init(0.9, 0.999, stream=s)
        plan.accumulate(0, first=True, stream=s)        # acc = g = 0 (it is also the first moment)
        plan.grad_stats(scan=True, max_norm=0.0, stream=s)
        plan.adam_step(0.0, 1e-8, 0.0, stream=s)
        torch.cuda.synchronize()
        bad = 0
        for i in range(P // piece):
            sl = slice(i * piece, (i + 1) * piece)
            pat = patterns(i)
            ref = pat.view(torch.float32).to(tdt)
            got = p[sl]
            same = (got.view(torch.int16) == ref.view(torch.int16)) | (torch.isnan(ref) & torch.isnan(got))
            bad += int((~same).sum())
            # the master values themselves came back unchanged
            unchanged = (w[sl].view(torch.int32) == pat) | ~torch.isfinite(w[sl])
            assert bool(unchanged.all()), f"master changed in piece {i}"
        assert bad == 0, f"{bad} patterns differ"
        del w, z, v, p, g
    finally:
        plan.close()
        torch.cuda.empty_cache()


# ----------------------------------------------------------------------------
# degenerate layouts
# ----------------------------------------------------------------------------
def test_empty_plan_and_empty_tensors():
    s = torch.cuda.current_stream().cuda_stream
    with dp.Plan((), 2, "bf16", "bf16") as p:
        for role in ("param", "master", "exp_avg", "exp_avg_sq", "gbar"):
            p.bind(role, 0)
        for r in range(2):
            p.bind("acc", 0, r)
            p.bind("grad", 0, r)
        p.state_init(stream=s)
        p.accumulate(0, first=True, stream=s)
        p.accumulate(1, first=True, stream=s)
        p.reduce_replicas("acc", stream=s)
        p.grad_stats(scan=True, max_norm=1.0, stream=s)
        p.adam_step(1e-3, 1e-8, 0.0, stream=s)
        st = p.read_state(stream=s)
        assert st["t"] == 1 and st["found_inf"] == 0 and st["norm"] == 0.0
        # the bucket calls: one empty bucket covers [0, 0), so each completes at once
        p.accumulate_all_range(True, 0, 0, stream=s)
        p.accumulate_all_range(False, 0, 0, stream=s)
        p.reduce_replicas_range("acc", 0, 0, stream=s)
        p.grad_stats(scan=False, max_norm=1.0, stream=s)
        p.adam_step(1e-3, 1e-8, 0.0, stream=s)
        p.accumulate_reduce_range(0, 0, stream=s)
        p.grad_stats(scan=False, max_norm=1.0, stream=s)
        assert p.read_state(stream=s)["t"] == 3
    w = workloads.tiny().with_(numel=(0, 5000, 0, 0, 3, 0), n=2, a=2, steps=2)
    _full_parity(w, 2, label="zero-size tensors")


def test_single_pass_empty_plan():
    s = torch.cuda.current_stream().cuda_stream
    with dp.Plan((), 3, "bf16", "bf16") as p:
        for role in ("master", "exp_avg", "exp_avg_sq"):
            p.bind(role, 0, 0)
            p.bind(role, 0, 1)
        p.bind("param", 0)
        for r in range(3):
            p.bind("grad", 0, r)
        p.state_init(stream=s)
        p.reduce_adam_step(1e-3, 1e-8, 0.0, stream=s)
        st = p.read_state(stream=s)
        assert st["t"] == 1 and st["found_inf"] == 0 and st["norm"] == 0.0 and st["bank"] == 1
        p.reduce_adam_range(1e-3, 1e-8, 0.0, 0, 0, stream=s)  # one empty bucket covers [0, 0)
        p.reduce_adam_finish(stream=s)
        st = p.read_state(stream=s)
        assert st["t"] == 2 and st["bank"] == 0


def test_empty_shard_is_a_noop():
    w = workloads.tiny().with_(numel=(10000,), n=1, a=1, steps=1)
    run = DeviceRun(w, shards=[(0, 0), (5000, 5000)])
    try:
        before = run.window(0, w.P)
        run.run(1)
        after = run.window(0, w.P)
        for k in ("w", "m", "v", "p"):
            assert np.array_equal(before[k], after[k])
        assert run.states[0]["t"] == 1
    finally:
        run.close()
