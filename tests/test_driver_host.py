"""Host logic of the step driver (no GPU): the backward-order buckets and
the even shard ranges."""
import pytest

driver = pytest.importorskip("gradient_reduce_adam_amd.driver")

from synth import workloads  # noqa: E402


@pytest.mark.parametrize("mb", [0.001, 1, 4, 16, 64, 1 << 20])
def test_backward_buckets_tile_the_space_in_reverse(mb):
    w = workloads.gpt2_small()
    off = [int(x) for x in w.offsets]
    bb = int(mb * (1 << 20))
    buckets = driver.backward_buckets(w.numel, bb)
    # contiguous, from the end of the flat space back to 0
    assert buckets[0][1] == w.P and buckets[-1][0] == 0
    for (lo, hi), (lo2, hi2) in zip(buckets, buckets[1:]):
        assert hi2 == lo and lo2 < hi2
    starts = set(off)
    for i, (lo, hi) in enumerate(buckets):
        assert lo in starts and hi in starts  # whole tensors only
        if i < len(buckets) - 1:  # every bucket but the last reaches the size
            assert 2 * (hi - lo) >= bb
            # and closes at the first tensor that reaches it
            inner = [t for t in range(len(off) - 1) if lo < off[t] < hi]
            for t in inner:
                assert 2 * (hi - off[t]) < bb


def test_backward_buckets_skip_empty_tensors():
    buckets = driver.backward_buckets((0, 5, 0, 0, 7, 0), 1)
    assert buckets == [(5, 12), (0, 5)]
    assert driver.backward_buckets((), 1) == []


def test_even_shards_tile():
    for P, k in ((10, 3), (7, 8), (0, 2), (124439808, 8)):
        sh = driver.even_shards(P, k)
        assert len(sh) == k and sh[0][0] == 0 and sh[-1][1] == P
        assert all(a[1] == b[0] for a, b in zip(sh, sh[1:]))
        assert max(e - b for b, e in sh) - min(e - b for b, e in sh) <= 1


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: any other --gpus value exits with status 2
    and a message, before anything is allocated."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""
