"""Checkpoints on the host (no GPU): the shard files, the manifest and its
atomic commit, resharded reads, integrity checks, and a recovery drill where
the writer is killed mid-checkpoint.  Everything here goes through the host
layer of the C ABI (dpckpt.h) with numpy arrays."""
import os
import signal
import subprocess
import sys
import textwrap
import time

import numpy as np
import pytest

dp = pytest.importorskip("gradient_reduce_adam_amd")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NUMEL = (1000003, 17, 2 * (1 << 20) + 5, 1, 300000)  # ragged; several checksum blocks per shard
P = sum(NUMEL)
CFG = dict(beta1=0.9, beta2=0.999, scaler_mode=2, growth_interval=2000, init_scale=65536.0, backoff=0.5, growth=2.0)


def _state(seed, n=P):
    rng = np.random.default_rng(seed)
    return {"master": rng.standard_normal(n).astype(np.float32),
            "exp_avg": rng.standard_normal(n).astype(np.float32) * 1e-3,
            "exp_avg_sq": rng.random(n).astype(np.float32) * 1e-6,
            "param": rng.integers(0, 1 << 16, n, dtype=np.uint64).astype(np.uint16)}


def _scalars(t):
    return dict(t=t, iter=t + 1, growth_tracker=t, beta1_pow=0.9 ** t, beta2_pow=0.999 ** t, scale=32768.0,
                found_inf=0, bank=0, sumsq=1.25, norm=float("nan"), clip=1.0, gscale=1.0 / 32768.0)


def _cuts(k, seed=0):
    rng = np.random.default_rng(seed)
    inner = sorted(rng.choice(np.arange(1, P), size=k - 1, replace=False).tolist())
    c = [0] + inner + [P]
    return list(zip(c[:-1], c[1:]))


def _save(d, gen, st, shards, pdt="bf16", scal=None):
    for b, e in shards:
        dp.dp_ckpt_write_shard(str(d), gen, NUMEL, pdt, b, e, st["master"][b:e], st["exp_avg"][b:e],
                               st["exp_avg_sq"][b:e], st["param"][b:e])
    dp.dp_ckpt_commit(str(d), gen, NUMEL, pdt, scal or _scalars(gen), CFG)


def _assert_range(d, st, b, e, pdt="bf16"):
    got = dp.dp_ckpt_read(str(d), NUMEL, pdt, b, e)
    for k in ("master", "exp_avg", "exp_avg_sq", "param"):
        assert np.array_equal(got[k].view(np.uint8), st[k][b:e].view(np.uint8)), (k, b, e)
    return got


def test_round_trip_and_resharding(tmp_path):
    st = _state(1)
    _save(tmp_path, 1, st, _cuts(8, seed=1))
    # read back as 4 other shards, as the whole range, and as ranges across shard and block edges
    for b, e in _cuts(4, seed=2) + [(0, P), (0, 1), (P - 1, P), ((1 << 20) - 3, (1 << 20) + 3), (5, 5)]:
        _assert_range(tmp_path, st, b, e)
    got = dp.dp_ckpt_read(str(tmp_path), NUMEL, "bf16", 0, 0, arrays=False)
    want = _scalars(1)
    for k, v in want.items():
        if k == "bank":
            continue
        g = got["scalars"][k]
        assert (np.isnan(g) and np.isnan(v)) or g == v, k  # exact bits, NaN included
    assert got["cfg"] == CFG and got["generation"] == 1


def test_empty_shards_and_empty_layout(tmp_path):
    st = _state(2)
    _save(tmp_path, 0, st, [(0, 0), (0, 500), (500, 500), (500, P), (P, P)])
    _assert_range(tmp_path, st, 0, P)
    e = tmp_path / "empty"
    e.mkdir()
    dp.dp_ckpt_commit(str(e), 0, (), "f16", _scalars(0), CFG)
    assert dp.dp_ckpt_read(str(e), (), "f16", 0, 0)["generation"] == 0


def test_commit_needs_an_exact_tiling(tmp_path):
    st = _state(3)
    for b, e in [(0, 1000), (2000, P)]:  # a gap
        dp.dp_ckpt_write_shard(str(tmp_path), 5, NUMEL, "bf16", b, e, st["master"][b:e], st["exp_avg"][b:e],
                               st["exp_avg_sq"][b:e], st["param"][b:e])
    with pytest.raises(dp.DpError) as ex:
        dp.dp_ckpt_commit(str(tmp_path), 5, NUMEL, "bf16", _scalars(5), CFG)
    assert ex.value.status == dp.DP_ERR_STATE and "gap" in ex.value.message
    b, e = 500, 2500  # now an overlap
    dp.dp_ckpt_write_shard(str(tmp_path), 5, NUMEL, "bf16", b, e, st["master"][b:e], st["exp_avg"][b:e],
                           st["exp_avg_sq"][b:e], st["param"][b:e])
    with pytest.raises(dp.DpError) as ex:
        dp.dp_ckpt_commit(str(tmp_path), 5, NUMEL, "bf16", _scalars(5), CFG)
    assert ex.value.status == dp.DP_ERR_STATE and "overlap" in ex.value.message
    with pytest.raises(dp.DpError) as ex:  # nothing was committed
        dp.dp_ckpt_read(str(tmp_path), NUMEL, "bf16", 0, 10)
    assert ex.value.status == dp.DP_ERR_STATE


def test_argument_and_layout_errors(tmp_path):
    st = _state(4)
    with pytest.raises(dp.DpError) as ex:
        dp.dp_ckpt_write_shard(str(tmp_path), 1, NUMEL, "bf16", 5, P + 1, *[np.zeros(P - 4, t) for t in
                                                                            (np.float32,) * 3 + (np.uint16,)])
    assert ex.value.status == dp.DP_ERR_RANGE
    with pytest.raises(dp.DpError) as ex:
        dp.dp_ckpt_write_shard(str(tmp_path / "missing"), 1, NUMEL, "bf16", 0, 10, st["master"][:10],
                               st["exp_avg"][:10], st["exp_avg_sq"][:10], st["param"][:10])
    assert ex.value.status == dp.DP_ERR_IO
    _save(tmp_path, 1, st, [(0, P)])
    for numel, pdt in [(NUMEL[:-1] + (NUMEL[-1] + 1,), "bf16"), ((P,), "bf16"), (NUMEL, "f16")]:
        with pytest.raises(dp.DpError) as ex:
            dp.dp_ckpt_read(str(tmp_path), numel, pdt, 0, 10)
        assert ex.value.status == dp.DP_ERR_BAD_LAYOUT
    with pytest.raises(dp.DpError) as ex:
        dp.dp_ckpt_read(str(tmp_path), NUMEL, "bf16", 10, P + 1)
    assert ex.value.status == dp.DP_ERR_RANGE


def _flip(path, offset):
    with open(path, "r+b") as f:
        f.seek(offset)
        b = f.read(1)
        f.seek(offset)
        f.write(bytes([b[0] ^ 0x40]))


def test_corruption_is_detected_block_by_block(tmp_path):
    st = _state(5)
    _save(tmp_path, 3, st, [(0, P)])
    shard = tmp_path / f"g3-0-{P}.dpshard"
    # the second array (m) starts on a 4096-byte boundary after the header,
    # the checksum table and the master array
    nblocks = (P + (1 << 20) - 1) >> 20
    up = lambda x: (x + 4095) // 4096 * 4096
    m_off = up(up(256 + 4 * nblocks * 8) + 4 * P)
    bad_elem = 2 * (1 << 20) + 7  # inside block 2 of m
    _flip(shard, m_off + 4 * bad_elem)
    _assert_range(tmp_path, st, 0, 2 * (1 << 20))  # blocks 0-1 are intact
    with pytest.raises(dp.DpError) as ex:
        dp.dp_ckpt_read(str(tmp_path), NUMEL, "bf16", bad_elem, bad_elem + 1)
    assert ex.value.status == dp.DP_ERR_CORRUPT and "checksum" in ex.value.message
    # a damaged header, a truncated file and a damaged manifest
    _save(tmp_path, 4, st, [(0, P)])
    shard = tmp_path / f"g4-0-{P}.dpshard"
    _flip(shard, 20)
    with pytest.raises(dp.DpError) as ex:
        dp.dp_ckpt_read(str(tmp_path), NUMEL, "bf16", 0, 1)
    assert ex.value.status == dp.DP_ERR_CORRUPT
    _save(tmp_path, 5, st, [(0, P)])
    shard = tmp_path / f"g5-0-{P}.dpshard"
    os.truncate(shard, os.path.getsize(shard) - 4096)
    with pytest.raises(dp.DpError) as ex:
        dp.dp_ckpt_read(str(tmp_path), NUMEL, "bf16", 0, 1)
    assert ex.value.status == dp.DP_ERR_CORRUPT
    _save(tmp_path, 6, st, [(0, P)])
    _flip(tmp_path / "manifest.dpck", 30)
    with pytest.raises(dp.DpError) as ex:
        dp.dp_ckpt_read(str(tmp_path), NUMEL, "bf16", 0, 1)
    assert ex.value.status == dp.DP_ERR_CORRUPT


def test_generations(tmp_path):
    a, b = _state(6), _state(7)
    _save(tmp_path, 1, a, _cuts(3, seed=3))
    # generation 2 written in part, not committed: readers still see generation 1
    for lo, hi in _cuts(5, seed=4)[:3]:
        dp.dp_ckpt_write_shard(str(tmp_path), 2, NUMEL, "bf16", lo, hi, b["master"][lo:hi], b["exp_avg"][lo:hi],
                               b["exp_avg_sq"][lo:hi], b["param"][lo:hi])
    assert _assert_range(tmp_path, a, 0, P)["generation"] == 1
    # finished and committed: generation 2 replaces generation 1, whose files go
    for lo, hi in _cuts(5, seed=4)[3:]:
        dp.dp_ckpt_write_shard(str(tmp_path), 2, NUMEL, "bf16", lo, hi, b["master"][lo:hi], b["exp_avg"][lo:hi],
                               b["exp_avg_sq"][lo:hi], b["param"][lo:hi])
    dp.dp_ckpt_commit(str(tmp_path), 2, NUMEL, "bf16", _scalars(2), CFG)
    assert _assert_range(tmp_path, b, 0, P)["generation"] == 2
    assert not [f for f in os.listdir(tmp_path) if f.startswith("g1-")]


WRITER = textwrap.dedent("""
    import sys
    import numpy as np
    sys.path.insert(0, {root!r})
    import gradient_reduce_adam_amd as dp
    d, numel = sys.argv[1], {numel!r}
    P = sum(numel)
    rng = np.random.default_rng(99)
    st = [rng.standard_normal(P).astype(np.float32) for _ in range(3)] + [np.zeros(P, np.uint16)]
    cuts = [P * i // 8 for i in range(9)]
    print("writing", flush=True)
    while True:  # generation 2 over and over, never committed, until killed
        for b, e in zip(cuts[:-1], cuts[1:]):
            dp.dp_ckpt_write_shard(d, 2, numel, "bf16", b, e, *[a[b:e] for a in st])
""")


def test_writer_killed_mid_checkpoint_leaves_the_last_commit_whole(tmp_path):
    """Recovery drill: a writer is killed (SIGKILL) while it writes the next
    generation; the directory still reads back the last committed generation
    bit for bit, and the next commit clears the debris."""
    st = _state(8)
    _save(tmp_path, 1, st, _cuts(8, seed=5))
    code = WRITER.format(root=ROOT, numel=NUMEL)
    proc = subprocess.Popen([sys.executable, "-c", code, str(tmp_path)], stdout=subprocess.PIPE,
                            stderr=subprocess.STDOUT)
    try:
        assert proc.stdout.readline().strip() == b"writing"
        deadline = time.time() + 60
        while time.time() < deadline:  # wait until it is inside a write
            if any(f.startswith(".tmp-g2-") for f in os.listdir(tmp_path)):
                break
            time.sleep(0.002)
        time.sleep(0.05)
    finally:
        proc.send_signal(signal.SIGKILL)
        proc.wait(timeout=30)
    debris = [f for f in os.listdir(tmp_path) if f.startswith(".tmp-g2-") or f.startswith("g2-")]
    assert debris, "the writer was killed before it wrote anything"
    got = _assert_range(tmp_path, st, 0, P)
    assert got["generation"] == 1
    # the next generation commits over the debris and removes it
    st3 = _state(9)
    _save(tmp_path, 3, st3, _cuts(2, seed=6))
    _assert_range(tmp_path, st3, 0, P)
    left = sorted(f for f in os.listdir(tmp_path) if f != "manifest.dpck")
    assert all(f.startswith("g3-") for f in left), left
