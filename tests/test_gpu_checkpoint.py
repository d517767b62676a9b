"""Checkpoint and resume on the GPU, through the C ABI: the recovery drill.
A run is interrupted after some steps, saved shard by shard, and restored
over a different partition of the flat parameter space (8 shards come back
as 4, or 3 as 1).  It then finishes its steps.  The result must equal the
uninterrupted run bit for bit -- state, parameters and every scalar --
and so match the oracle's uninterrupted run under the stated tolerances."""
import numpy as np
import pytest
import torch

import gradient_reduce_adam_amd as dp
from synth import workloads

from gpu_common import DeviceRun, assert_scalars_match, assert_state_close, log, oracle_run, ulp_bound

pytestmark = pytest.mark.gpu

RAGGED = (3000, 17, 4096, 5, 70001, 256, 1, 65536, 131075)


def _ranges(P, k):
    cuts = [P * i // k for i in range(k + 1)]
    return list(zip(cuts[:-1], cuts[1:]))


def _snapshot(run):
    torch.cuda.synchronize()
    return run.window(0, run.w.P), run.d.read_state()


def _same(a, b, where):
    (sa, xa), (sb, xb) = a, b
    for k in ("w", "m", "v", "p"):
        assert np.array_equal(sa[k].view(np.uint8), sb[k].view(np.uint8)), f"{where}: {k}"
    keys = [k for k in xa if k != "bank"]
    assert np.array_equal(np.array([xa[k] for k in keys], np.float64).view(np.uint64),
                          np.array([xb[k] for k in keys], np.float64).view(np.uint64)), f"{where}: scalars"


CASES = {
    # ZeRO-style update over 8 shards, restored as 4; dynamic scale that grows,
    # non-finite gradients after the restore
    "dynamic_partials_8_to_4": dict(base="zero3_rank_7b", numel=RAGGED, n=4, a=1, growth_interval=2, steps=6,
                                    save_at=3, save_shards=8, load_shards=4,
                                    injections=((2, 1, 1, 5, float("nan")), (5, 0, 1, 7000, float("inf")))),
    # clipping, three replicas with two micro-steps, 3 shards restored as 1
    "bf16_clip_3_to_1": dict(base="gpt2_small", numel=RAGGED, n=3, a=2, max_norm=0.05, scaled_tensors=(4,),
                             steps=4, save_at=2, save_shards=3, load_shards=1),
    # the single pass: the state lives in whichever bank is current when saved
    "single_pass_banks": dict(base="tiny", numel=RAGGED, n=4, a=2, steps=5, save_at=3, save_shards=5,
                              load_shards=2, single=True),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_recovery_drill_resharded_bitwise(name, tmp_path):
    spec = dict(CASES[name])
    base = workloads.by_name(spec.pop("base"))
    steps, save_at = spec.pop("steps"), spec.pop("save_at")
    ks, kl = spec.pop("save_shards"), spec.pop("load_shards")
    single = spec.pop("single", False)
    w = base.with_(**spec)
    P = w.P
    log(f"recovery drill {name}: P={P} steps={steps} save after {save_at}, {ks} shards -> {kl}")
    save_sh = None if single else _ranges(P, ks)
    load_sh = None if single else _ranges(P, kl)
    # uninterrupted
    run = DeviceRun(w, shards=save_sh, single_pass=single)
    try:
        run.run(steps)
        whole = _snapshot(run)
    finally:
        run.close()
    # interrupted after save_at steps, saved over ks ranges
    run = DeviceRun(w, shards=save_sh, single_pass=single)
    try:
        run.run(save_at)
        run.d.save_checkpoint(str(tmp_path), save_at, ranges=_ranges(P, ks))
        at_save = _snapshot(run)
    finally:
        run.close()
    # a fresh process state: new plan and buffers, restored over kl ranges
    run = DeviceRun(w, shards=load_sh, single_pass=single)
    try:
        st = run.d.load_checkpoint(str(tmp_path), ranges=_ranges(P, kl))
        assert st["iter"] == save_at and st["bank"] == 0
        _same(_snapshot(run), at_save, f"{name} right after the restore")
        for _ in range(steps - save_at):
            run.step()
        _same(_snapshot(run), whole, f"{name} at the end")
    finally:
        run.close()
    # the oracle's uninterrupted run agrees with the resumed one
    ref = oracle_run(w, steps)
    assert_scalars_match(whole[1], ref.scalars[-1], where=name)
    assert_state_close(whole[0], ref.state[(0, P)], ulp_bound(w), where=name)


def test_save_and_load_through_per_tensor_bindings(tmp_path):
    """Save from flat buffers, restore into misaligned per-tensor buffers
    (copies per tensor piece), save again from those, and read both
    checkpoints back on the host: the same bits everywhere."""
    w = workloads.tiny().with_(numel=(1001, 4099, 65536 + 3, 7), n=2, a=1, steps=2)
    P, off, T = w.P, w.offsets, w.T
    run = DeviceRun(w)
    try:
        run.run(2)
        (tmp_path / "a").mkdir()
        run.d.save_checkpoint(str(tmp_path / "a"), 2, ranges=_ranges(P, 3))
        flat = _snapshot(run)
    finally:
        run.close()
    plan = dp.Plan(w.numel, w.n, w.grad_dtype, w.param_dtype)
    s = torch.cuda.current_stream().cuda_stream
    backs = []

    def shifted(dtype):
        back = torch.full((P + 2 * T,), 7, dtype=dtype, device="cuda")
        backs.append(back)
        return [back[int(off[t]) + 2 * t + 1:int(off[t + 1]) + 2 * t + 1] for t in range(T)]

    try:
        roles = {r: shifted(torch.float32) for r in ("master", "exp_avg", "exp_avg_sq")}
        roles["param"] = shifted(torch.float16)
        for r, ts in roles.items():
            plan.bind_tensors(r, ts)
        plan.state_init(w.beta1, w.beta2, stream=s)
        for b, e in _ranges(P, 4):
            plan.checkpoint_load(str(tmp_path / "a"), b, e, restore_scalars=True, stream=s)
        torch.cuda.synchronize()
        got = {k: torch.cat(roles[r]).cpu().numpy() for k, r in (("w", "master"), ("m", "exp_avg"),
                                                                   ("v", "exp_avg_sq"))}
        got["p"] = torch.cat(roles["param"]).view(torch.int16).cpu().numpy().view(np.uint16)
        for k in ("w", "m", "v", "p"):
            assert np.array_equal(got[k].view(np.uint8), flat[0][k].view(np.uint8)), k
        (tmp_path / "b").mkdir()
        for b, e in _ranges(P, 2):
            plan.checkpoint_save(str(tmp_path / "b"), 9, b, e, stream=s)
        plan.checkpoint_commit(str(tmp_path / "b"), 9, stream=s)
    finally:
        plan.close()
    ra = dp.dp_ckpt_read(str(tmp_path / "a"), w.numel, w.param_dtype, 0, P)
    rb = dp.dp_ckpt_read(str(tmp_path / "b"), w.numel, w.param_dtype, 0, P)
    for k in ("master", "exp_avg", "exp_avg_sq", "param"):
        assert np.array_equal(ra[k].view(np.uint8), rb[k].view(np.uint8)), k
    assert ra["scalars"]["t"] == rb["scalars"]["t"] == 2 and rb["generation"] == 9


def test_load_errors(tmp_path):
    w = workloads.tiny().with_(numel=(5000, 3), n=1, a=1, steps=1)
    run = DeviceRun(w)
    try:
        with pytest.raises(dp.DpError) as e:  # nothing committed yet
            run.d.plan.checkpoint_load(str(tmp_path), stream=run.stream)
        assert e.value.status == dp.DP_ERR_STATE
        run.run(1)
        run.d.save_checkpoint(str(tmp_path), 1)
    finally:
        run.close()
    other = w.with_(numel=(5000, 4))
    run = DeviceRun(other)
    try:
        with pytest.raises(dp.DpError) as e:
            run.d.plan.checkpoint_load(str(tmp_path), stream=run.stream)
        assert e.value.status == dp.DP_ERR_BAD_LAYOUT
    finally:
        run.close()
    run = DeviceRun(w.with_(beta2=0.99))
    try:
        before = _snapshot(run)
        with pytest.raises(dp.DpError) as e:
            run.d.plan.checkpoint_load(str(tmp_path), restore_scalars=True, stream=run.stream)
        assert e.value.status == dp.DP_ERR_STATE and "optimizer settings" in e.value.message
        # the mismatch is found before anything is written
        _same(_snapshot(run), before, "after a refused restore")
    finally:
        run.close()


def test_offloaded_state_round_trip(tmp_path):
    """A run whose state lives in pinned host memory saves a checkpoint that
    an HBM-resident run restores, and both finish with the same bits as an
    uninterrupted run."""
    w = workloads.tiny().with_(numel=RAGGED, n=2, a=2, steps=4)
    P = w.P
    run = DeviceRun(w)
    try:
        run.run(4)
        whole = _snapshot(run)
    finally:
        run.close()
    run = DeviceRun(w, state_location="host")
    try:
        run.run(2)
        run.d.save_checkpoint(str(tmp_path), 2, ranges=_ranges(P, 3))
    finally:
        run.close()
    run = DeviceRun(w)
    try:
        run.d.load_checkpoint(str(tmp_path), ranges=_ranges(P, 2))
        run.step()
        run.step()
        _same(_snapshot(run), whole, "offloaded save, HBM restore")
    finally:
        run.close()


def test_partial_restore_goes_into_the_current_bank(tmp_path):
    """A single-pass run whose current bank is 1 restores only the first half
    of its range from a checkpoint taken a step earlier (when bank 0 was
    current): that half equals the checkpoint, the other half keeps the
    current bank's values, and bank 1 stays current."""
    w = workloads.tiny().with_(numel=RAGGED, n=2, a=1, steps=3)
    P, h = w.P, 131072 + 3000  # a cut inside a tensor
    run = DeviceRun(w, single_pass=True)
    try:
        run.run(2)
        run.d.save_checkpoint(str(tmp_path), 2, ranges=_ranges(P, 3))
        saved, saved_st = _snapshot(run)
        assert saved_st["bank"] == 0
        run.step()
        before, before_st = _snapshot(run)
        assert before_st["bank"] == 1
        run.d.plan.checkpoint_load(str(tmp_path), 0, h, restore_scalars=False, stream=run.stream)
        after, after_st = _snapshot(run)
        assert after_st["bank"] == 1 and after_st["t"] == before_st["t"]
        for k in ("w", "m", "v", "p"):
            assert np.array_equal(after[k][:h].view(np.uint8), saved[k][:h].view(np.uint8)), k
            assert np.array_equal(after[k][h:].view(np.uint8), before[k][h:].view(np.uint8)), k
            assert not np.array_equal(saved[k][h:].view(np.uint8), before[k][h:].view(np.uint8)), k
    finally:
        run.close()


def _random_ranges(rng, P):
    """A random partition of [0, P) into 1-8 ranges with arbitrary cuts (empty
    ranges included)."""
    cuts = sorted([0, P] + [int(x) for x in rng.integers(0, P + 1, int(rng.integers(0, 8)))])
    return list(zip(cuts[:-1], cuts[1:]))


@pytest.mark.parametrize("seed", range(8))
def test_random_recovery_drills_bitwise(seed, tmp_path):
    """Seeded drills: a random ragged layout, update path (two-pass with
    clipping or a dynamic scale, or the single pass whose current bank is
    either), interruption point, and save and restore partitions with
    arbitrary cuts.  The resumed run equals the uninterrupted one bit for bit."""
    rng = np.random.default_rng(7000 + seed)
    T = int(rng.integers(1, 12))
    numel = tuple(int(x) for x in rng.integers(0, 30000, T))
    if sum(numel) == 0:
        numel = (5000,)
    single = bool(rng.random() < 0.5)
    base = workloads.tiny() if single else workloads.gpt2_small()
    spec = dict(numel=numel, n=int(rng.integers(1, 5)), a=int(rng.integers(1, 4)), steps=int(rng.integers(3, 6)))
    if not single:
        spec.update(max_norm=float(rng.choice([0.0, 0.05])), scaled_tensors=())
    if rng.random() < 0.5:
        spec.update(scaler="dynamic", init_scale=256.0, growth_interval=2)
    w = base.with_(**spec)
    P, steps = w.P, w.steps
    save_at = int(rng.integers(1, steps))
    save_r, load_r = _random_ranges(rng, P), _random_ranges(rng, P)
    log(f"drill {seed}: P={P} T={T} n={w.n} a={w.a} single={single} clip={w.max_norm} scaler={w.scaler} "
        f"steps={steps} save after {save_at} as {len(save_r)}, restore as {len(load_r)}")
    run = DeviceRun(w, single_pass=single)
    try:
        run.run(steps)
        whole = _snapshot(run)
    finally:
        run.close()
    run = DeviceRun(w, single_pass=single)
    try:
        run.run(save_at)
        run.d.save_checkpoint(str(tmp_path), save_at, ranges=save_r)
    finally:
        run.close()
    run = DeviceRun(w, single_pass=single)
    try:
        if single and save_at % 2 == 1:  # restore into a plan whose bank 1 is current
            run.run(1)
        st = run.d.load_checkpoint(str(tmp_path), ranges=load_r)
        assert st["iter"] == save_at
        for _ in range(steps - save_at):
            run.step()
        _same(_snapshot(run), whole, f"drill {seed}")
    finally:
        run.close()
