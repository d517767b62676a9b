"""The offloaded optimizer state: master, m and v in pinned host memory,
read and written by the same update kernels across PCIe.  Same bits as the
state in HBM, so the oracle agrees too."""
import numpy as np
import pytest

from synth import workloads

from gpu_common import DeviceRun, assert_scalars_match, assert_state_close, log, oracle_run, ulp_bound

pytestmark = pytest.mark.gpu

RAGGED = (3000, 17, 4096, 5, 70001, 256, 1, 65536, 131075)

CASES = {
    "clip_two_pass": (dict(base="gpt2_small", numel=RAGGED, n=3, a=2, max_norm=0.05, scaled_tensors=(4,)), 3, False),
    "partials_single_pass": (dict(base="zero3_rank_7b", numel=RAGGED, n=4, a=1, growth_interval=2,
                                  injections=((2, 1, 1, 70000, float("inf")),)), 4, True),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_host_state_equals_hbm_state_bitwise(name):
    spec, steps, single = CASES[name]
    spec = dict(spec)
    w = workloads.by_name(spec.pop("base")).with_(**spec)
    log(f"offload {name}: P={w.P} steps={steps} single_pass={single}")
    outs = []
    for loc in ("hbm", "host"):
        run = DeviceRun(w, single_pass=single, state_location=loc)
        try:
            if loc == "host":
                assert not run.d.master.is_cuda and run.d.master.is_pinned()
            st = run.run(steps)
            outs.append((run.window(0, w.P), st))
        finally:
            run.close()
    (a, sa), (b, sb) = outs
    for k in ("w", "m", "v", "p"):
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k
    for x, y in zip(sa, sb):
        assert np.array_equal(np.array(list(x.values()), np.float64).view(np.uint64),
                              np.array(list(y.values()), np.float64).view(np.uint64))
    ref = oracle_run(w, steps)
    assert_scalars_match(sb[-1], ref.scalars[-1], where=name)
    assert_state_close(b, ref.state[(0, w.P)], ulp_bound(w), where=name)


def test_staged_offload_equals_direct_bitwise():
    """The staged variant (state copied through device slots on two copy
    streams) gives the same bits as the direct one; pieces smaller than a
    tensor and a shard boundary inside a piece's range exercise the
    rebinding."""
    w = workloads.gpt2_small().with_(numel=RAGGED, n=2, a=2, max_norm=0.05, scaled_tensors=(4,))
    shards = [(0, 100003), (100003, w.P)]
    outs = []
    for off in ("direct", "staged"):
        run = DeviceRun(w, shards=shards, state_location="host", offload=off, stage_elems=65536)
        try:
            st = run.run(4)
            outs.append((run.window(0, w.P), st))
        finally:
            run.close()
    (a, sa), (b, sb) = outs
    for k in ("w", "m", "v", "p"):
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k
    assert [x["t"] for x in sa] == [x["t"] for x in sb]
