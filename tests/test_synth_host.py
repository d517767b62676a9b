"""The seeded input generator (host twin) and the workload layouts."""
import numpy as np
import pytest

import oracle
import synth
from synth import workloads


def test_splitmix64_published_first_output():
    # SplitMix64 seeded with 0 advances its state by GOLDEN and outputs
    # mix64(GOLDEN) = 0xE220A8397B1DCDAF (Vigna's reference splitmix64.c).
    assert synth.mix64(synth.GOLDEN) == 0xE220A8397B1DCDAF
    assert synth.host_hash_at(0, 0) == 0xE220A8397B1DCDAF


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_host_twin_matches_python_definition(dtype):
    rng = np.random.default_rng(7)
    for _ in range(4):
        key = synth.stream_key(int(rng.integers(0, 1 << 40)), 2, int(rng.integers(1, 30)), int(rng.integers(0, 8)),
                               int(rng.integers(1, 9)))
        start = int(rng.integers(0, 1 << 34))
        for c in (synth.scale_constant(1e-3), synth.scale_constant(1e-4, 1.0, 65536.0),
                  synth.scale_constant(1e-4, 1.0, 1024.0), np.float32(1e-12), np.float32(1e31)):
            a = synth.py_normal(key, start, 500, c, dtype) if dtype != "f16" else None
            if dtype == "f16":
                with np.errstate(over="ignore"):
                    a = synth.py_normal(key, start, 500, c, dtype)
            b = synth.host_normal(key, start, 500, c, dtype, threads=3)
            assert a.tobytes() == b.tobytes()


def test_stream_keys_match_between_twins():
    for args in [(1, 1, 0, 0, 0), (2, 2, 20, 7, 8), (5, 2, 3, 3, 4), (3, 3, 0, 0, 0)]:
        assert synth.stream_key(*args) == synth.host_stream_key(*args)


def test_irwin_hall_moments():
    n = 1 << 22
    x = synth.host_normal(synth.stream_key(9, 2, 1, 0, 1), 0, n, synth.scale_constant(1.0), "f32", threads=4)
    assert abs(x.mean()) < 4 / np.sqrt(n)
    assert abs(x.std() - 1.0) < 4 / np.sqrt(n)
    assert np.abs(x).max() <= 2 * np.sqrt(3.0) + 1e-6  # Irwin-Hall(4) support


def test_workload_layouts():
    g = workloads.gpt2_small()
    assert g.T == 148 and g.P == 124_439_808
    assert len(g.scaled_tensors) == 2
    assert oracle.global_batch(4, g.n, g.a) == 256
    s = workloads.unsharded_7b()
    assert s.T == 225 and s.P == 6_607_077_376
    z = workloads.zero3_rank_7b()
    assert z.P == 875_000_000 and z.P * 8 == 7_000_000_000
    t = workloads.tp_column_slice()
    assert t.P == 1 << 32 and 131072 * 262144 // 8 == t.P
    assert workloads.tiny().P == 1 << 20


def test_grad_segments_cover_range_and_scale_only_selected_tensors():
    w = workloads.gpt2_small()
    off = w.offsets
    lo, hi = int(off[3]) - 5, int(off[6]) + 9
    segs = list(workloads.grad_segments(w, lo, hi, 1.0))
    assert segs[0][0] == lo and sum(c for _, c, _ in segs) == hi - lo
    base = synth.scale_constant(w.grad_sigma)
    for start, count, c in segs:
        t = int(np.searchsorted(off, start, side="right") - 1)
        assert (c != base) == (t in w.scaled_tensors)


def test_loss_scale_is_exact_power_of_two_scaling():
    w = workloads.zero3_rank_7b().with_(numel=(100000,))
    a = synth.grad_host(w, 1, 0, 1, 0, w.P, 65536.0)
    b = synth.grad_host(w, 1, 0, 1, 0, w.P, 32768.0)
    fa = oracle.widen(a, "bf16")
    fb = oracle.widen(b, "bf16")
    assert np.array_equal(fa, fb * 2)


def test_injection_written_on_host():
    w = workloads.zero3_rank_7b().with_(numel=(1000,), injections=((3, 0, 1, 500, float("inf")),))
    g = synth.grad_host(w, 3, 0, 1, 0, 1000, 65536.0)
    assert g[500] == 0x7F80
    assert np.isfinite(oracle.widen(synth.grad_host(w, 3, 1, 1, 0, 1000, 65536.0), "bf16")).all()
