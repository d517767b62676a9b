"""One whole step captured into a HIP graph and replayed: every replay,
with the program's own eager work (new gradients, a state read-back) in
between, gives the same bits as the eager step sequence."""
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
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_graph_replays_equal_eager_steps(name):
    spec, single = CASES[name]
    spec = dict(spec)
    w = workloads.by_name(spec.pop("base")).with_(**spec)
    steps = 5
    log(f"graph {name}: P={w.P} n={w.n} a={w.a} single_pass={single}")
    eager = DeviceRun(w, single_pass=single)
    try:
        ref_states = eager.run(steps)
        ref = eager.window(0, w.P)
    finally:
        eager.close()
    last = 1 if w.partials else w.a
    run = DeviceRun(w, single_pass=single, stream=torch.cuda.Stream())
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
