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


@pytest.mark.parametrize("numel,mb", [((875000000,), 64), ((3000, 17, 70001, 256, 131075), 0.05),
                                      ((5, 1 << 20, 7, 1 << 21, 3), 1), ((), 1), ((300, 0, 1000), 0.0001)])
def test_split_backward_buckets_tile_on_the_piece_grid(numel, mb):
    bb = int(mb * (1 << 20))
    step = max(256, (bb // 2) // 256 * 256)
    off = [0]
    for x in numel:
        off.append(off[-1] + x)
    buckets = driver.backward_buckets(numel, bb, split=True)
    if not numel or off[-1] == 0:
        assert buckets == []
        return
    # contiguous, from the end of the flat space back to 0
    assert buckets[0][1] == off[-1] and buckets[-1][0] == 0
    for (lo, hi), (lo2, hi2) in zip(buckets, buckets[1:]):
        assert hi2 == lo and lo2 < hi2
    for lo, hi in buckets:
        for x in (lo, hi):  # a tensor boundary, or a multiple of 256 into a tensor
            t = max(i for i in range(len(numel)) if off[i] <= x) if x < off[-1] else len(numel)
            assert x == off[-1] or x == off[t] or (x - off[t]) % 256 == 0
        inside = [t for t in range(len(numel)) if off[t] <= lo < off[t + 1]]
        if inside and numel[inside[0]] * 2 > bb:  # a cut of a large tensor
            assert hi - lo <= step and hi <= off[inside[0] + 1]


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


@pytest.mark.parametrize("name,two_pass,single,unfused", [
    ("tiny", 82, 74, 114), ("gpt2_small", 610, 602, 674), ("zero3_rank_7b", 50, 42, 50),
    ("unsharded_7b", 106, 98, 106), ("tp_column_slice", 162, 154, 194)])
def test_bench_byte_model(name, two_pass, single, unfused):
    """The bytes per parameter and step that bench.py divides by the step
    time, against closed forms.  Unfused: the first micro-step writes the
    binary32 accumulator, every later one reads and writes it, the reduction
    reads it, g_bar is written and read back, and the update moves 30 B:
    n a (s_g + 8) + 34 with n >= 2 accumulators, a (s_g + 8) + 26 for one
    replica (g_bar is the accumulator), n s_g + 34 for incoming partials.
    This library fuses the last micro-step into the tree, so that
    accumulator is neither written back nor read again (8 B less per
    replica), and the single pass never stores g_bar (8 B less)."""
    import bench
    w = workloads.by_name(name)
    sg = 2
    if w.partials:
        ref_unfused = w.n * sg + 34
    elif w.n == 1:
        ref_unfused = w.a * (sg + 8) + 26
    else:
        ref_unfused = w.n * w.a * (sg + 8) + 34
    assert bench.unfused_bytes_per_param(w) == ref_unfused == unfused
    assert sum(bench.bytes_model(w, False).values()) == two_pass
    assert sum(bench.bytes_model(w, True).values()) == single == two_pass - 8
    if not w.partials and w.n > 1:
        assert unfused - two_pass == w.n * 8
