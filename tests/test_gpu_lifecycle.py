"""The plan's life cycle on the GPU, through the C ABI: a failed allocation of
the state leaves nothing behind and the plan usable for error reporting;
per-tensor pointer tables rebound between launches on a non-default stream
never reach a kernel that was launched with the old ones; and cached range
tables can be dropped when the shard partition changes during a run."""
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
