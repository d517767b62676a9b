"""One whole step captured into a HIP graph and replayed: every replay,
with the program's own eager work (new gradients, a state read-back) in
between, gives the same bits as the eager step sequence.  Replays launch on
the step's stream, so that work is ordered around them."""
import numpy as np
import pytest
import torch

import synth
from synth import workloads

from gpu_common import DeviceRun, log

pytestmark = pytest.mark.gpu

CASES = {
    # the tiny workload's shape, two-pass and single pass
    "tiny_two_pass": (dict(base="tiny", numel=(65536 * 3 + 7, 4099)), False),
    "tiny_single_pass": (dict(base="tiny", numel=(65536 * 3 + 7, 4099)), True),
    # clipping and a dynamic scale with a skipped step in the middle
    "clip_dynamic_skip": (dict(base="gpt2_small", numel=(3000, 17, 70001, 4096), n=3, a=2, max_norm=0.05,
                               scaled_tensors=(2,), scaler="dynamic", init_scale=1024.0, growth_interval=2,
                               injections=((3, 1, 2, 3100, float("inf")),)), False),
    # the state in pinned host memory: a replay that reads it across PCIe
    # takes long enough that a read of the state not ordered after it sees
    # the previous step
    "host_state_single_pass": (dict(base="tiny", numel=(65536 * 3 + 7, 4099), n=16, a=3, scaler="dynamic",
                                    init_scale=1024.0, growth_interval=2,
                                    injections=((1, 8, 1, 67706, float("inf")),)), True, "host"),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_graph_replays_equal_eager_steps(name):
    spec, single, *where = CASES[name]
    location = where[0] if where else "hbm"
    spec = dict(spec)
    w = workloads.by_name(spec.pop("base")).with_(**spec)
    steps = 5
    log(f"graph {name}: P={w.P} n={w.n} a={w.a} single_pass={single} state={location}")
    eager = DeviceRun(w, single_pass=single, state_location=location)
    try:
        ref_states = eager.run(steps)
        ref = eager.window(0, w.P)
    finally:
        eager.close()
    last = 1 if w.partials else w.a
    run = DeviceRun(w, single_pass=single, stream=torch.cuda.Stream(), state_location=location)
    d, st = run.d, run.d.stream.cuda_stream
    bufs = [[torch.empty(w.P, dtype=torch.int16, device="cuda") for _ in range(w.n)] for _ in range(last)]
    slots = [[b.data_ptr() for b in row] for row in bufs]

    def fill(step):  # eager work between replays: this step's gradients into the fixed buffers
        for k in range(1, last + 1):
            for r in range(w.n):
                synth.grad_device(w, step, r, k, slots[k - 1][r], d.scale, st)

    try:
        fill(1)
        d.issue_fixed(slots)  # step 1 eagerly: allocations and tables happen outside the capture
        s1 = d.read_state()
        d.scale = s1["scale"]
        assert s1["iter"] == 1
        fill(2)
        g = d.capture_step(slots)  # capturing runs nothing
        assert d.read_state()["iter"] == 1
        for step in range(2, steps + 1):
            if step > 2:
                fill(step)
            g.replay()
            s = d.read_state()
            d.scale = s["scale"]
            r = ref_states[step - 1]
            assert np.array_equal(np.array(list(s.values()), np.float64).view(np.uint64),
                                  np.array(list(r.values()), np.float64).view(np.uint64)), f"replay for step {step}"
        got = run.window(0, w.P)
        for k in ("w", "m", "v", "p"):
            assert np.array_equal(got[k].view(np.uint8), ref[k].view(np.uint8)), k
    finally:
        run.close()


def _bind_per_tensor(d, w):
    """Every role of the plan bound through per-tensor pointer tables into
    the memory it already holds."""
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


def test_graph_on_per_tensor_bindings():
    """A step on per-tensor pointer tables captured after one uncaptured step
    (which uploads the tables) replays with the eager sequence's bits; a
    capture that would have to upload a freshly rebound table is refused
    before anything is launched or recorded."""
    import gradient_reduce_adam_amd as dp

    w = workloads.by_name("gpt2_small").with_(numel=(3000, 17, 70001, 4096), n=2, a=2, max_norm=0.05,
                                              scaled_tensors=(2,))
    steps = 4
    eager = DeviceRun(w)
    try:
        ref_states = eager.run(steps)
        ref = eager.window(0, w.P)
    finally:
        eager.close()
    run = DeviceRun(w, stream=torch.cuda.Stream())
    d, st = run.d, run.d.stream.cuda_stream
    bufs = [[torch.empty(w.P, dtype=torch.int16, device="cuda") for _ in range(w.n)] for _ in range(w.a)]
    slots = [[b.data_ptr() for b in row] for row in bufs]

    def fill(step):
        for k in range(1, w.a + 1):
            for r in range(w.n):
                synth.grad_device(w, step, r, k, slots[k - 1][r], d.scale, st)

    try:
        _bind_per_tensor(d, w)
        fill(1)
        d.issue_fixed(slots)  # uncaptured: uploads every table
        d.scale = d.read_state()["scale"]
        # a rebound table is pending until an uncaptured call reads it: bind
        # the first moment to a copy of itself, try to capture, bind it back
        copy = d.exp_avg.clone()
        per = lambda t: [t.data_ptr() + 4 * int(o) for o in w.offsets[:-1]]  # noqa: E731
        torch.cuda.synchronize()
        d.plan.bind_tensors("exp_avg", per(copy), 0)
        with pytest.raises(dp.DpError) as e:
            d.capture_step(slots)
        assert e.value.status == dp.DP_ERR_STATE and "graph capture" in e.value.message
        torch.cuda.synchronize()
        assert d.read_state()["iter"] == 1
        d.plan.bind_tensors("exp_avg", per(d.exp_avg), 0)
        fill(2)
        d.issue_fixed(slots)  # uncaptured step 2 uploads it
        d.scale = d.read_state()["scale"]
        fill(3)
        g = d.capture_step(slots)
        for step in range(3, steps + 1):
            if step > 3:
                fill(step)
            g.replay()
            s = d.read_state()
            d.scale = s["scale"]
            r = ref_states[step - 1]
            assert np.array_equal(np.array(list(s.values()), np.float64).view(np.uint64),
                                  np.array(list(r.values()), np.float64).view(np.uint64)), f"replay for step {step}"
        got = run.window(0, w.P)
        for k in ("w", "m", "v", "p"):
            assert np.array_equal(got[k].view(np.uint8), ref[k].view(np.uint8)), k
    finally:
        run.close()
