"""Seeded random configurations of the whole step against the oracle, on the
GPU, through the C ABI.  Each seed draws a ragged tensor list (zero-size
tensors, tensors shorter than a piece, sizes off every alignment), the
replica and micro-step counts, the gradient and parameter formats, the chunk
size, clipping, the loss scaler with non-finite values injected, and the
update path (two-pass over random shard ranges, or the single pass when there
is no clipping).  The tolerances are the stated ones."""
import os

import numpy as np
import pytest

from synth import workloads

from gpu_common import DeviceRun, assert_scalars_match, assert_state_close, log, oracle_run, ulp_bound

pytestmark = pytest.mark.gpu


def _draw(seed):
    rng = np.random.default_rng(5000 + seed)
    T = int(rng.integers(1, 40))
    kinds = rng.integers(0, 4, T)
    numel = tuple(int(x) for x in np.where(kinds == 0, 0, np.where(kinds == 1, rng.integers(1, 256, T),
                                                np.where(kinds == 2, 256 * rng.integers(1, 64, T),
                                                         rng.integers(257, 40000, T)))))
    if sum(numel) == 0:
        numel = numel[:-1] + (1000,)
    n = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
    partials = n > 1 and rng.random() < 0.25
    a = 1 if partials else int(rng.integers(1, 5))
    gdt, pdt = str(rng.choice(["bf16", "f16"])), str(rng.choice(["bf16", "f16"]))
    clip = float(rng.choice([0.0, 0.0, 0.02, 1.0]))
    scaler = str(rng.choice(["none", "static", "dynamic"]))
    P = sum(numel)
    steps = int(rng.integers(2, 4))
    inj = ()
    if scaler != "none" or rng.random() < 0.5:
        s = int(rng.integers(1, steps + 1))
        inj = ((s, int(rng.integers(0, n)), int(rng.integers(1, a + 1)), int(rng.integers(0, P)),
                float(rng.choice([np.inf, -np.inf, np.nan]))),)
    base = workloads.zero3_rank_7b() if partials else workloads.gpt2_small()
    w = base.with_(numel=numel, n=n, a=a, grad_dtype=gdt, param_dtype=pdt, max_norm=clip, scaler=scaler,
                   init_scale=1024.0 if scaler != "none" else 1.0, growth_interval=2, partials=partials,
                   scaled_tensors=tuple(sorted(set(int(x) for x in rng.integers(0, T, 2)))), injections=inj,
                   grad_sigma=float(rng.choice([1e-4, 1e-3, 1e-2])), steps=steps)
    chunk = int(rng.choice([0, 256, 1024, 4096, 65536]))
    single = clip == 0.0 and rng.random() < 0.5
    shards = None
    if not single and rng.random() < 0.5:
        cuts = sorted(set([0, P] + [int(x) for x in rng.integers(0, P + 1, int(rng.integers(1, 5)))]))
        shards = list(zip(cuts[:-1], cuts[1:]))
    location = "host" if rng.random() < 0.25 else "hbm"  # the state offloaded to pinned host memory
    return w, chunk, single, shards, location


# DP_RANDOM_CONFIGS=N runs seeds 0 .. N-1 (default 32); 1851 and 3044 always
# run: clipped draws where m nearly cancels at one or two elements, beyond 64
# ulp and within the norm-order slack (gpu_common.m_slack)
SEEDS = sorted(set(range(int(os.environ.get("DP_RANDOM_CONFIGS", "32")))) | {1851, 3044})


@pytest.mark.parametrize("seed", SEEDS)
def test_random_configuration_matches_oracle(seed):
    w, chunk, single, shards, location = _draw(seed)
    log(f"seed {seed}: P={w.P} T={w.T} n={w.n} a={w.a} {w.grad_dtype}/{w.param_dtype} clip={w.max_norm} "
        f"scaler={w.scaler} partials={w.partials} chunk={chunk or 'default'} single={single} "
        f"shards={None if shards is None else len(shards)} injections={w.injections} state={location}")
    run = DeviceRun(w, shards=shards, chunk_elems=chunk, single_pass=single, state_location=location)
    try:
        states = run.run(w.steps)
        got = run.window(0, w.P)
    finally:
        run.close()
    ref = oracle_run(w, w.steps)
    for s, (g, r) in enumerate(zip(states, ref.scalars), start=1):
        assert_scalars_match(g, r, where=f"seed {seed} step {s}")
    rep = assert_state_close(got, ref.state[(0, w.P)], ulp_bound(w), where=f"seed {seed}")
    log(f"  max ulp: {rep}")
