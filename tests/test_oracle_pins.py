"""Pins of the CPU oracle against what the pages and the mathematics fix:
printed figures, hand-derived cases, closed forms, library routines for the
special cases that reduce to them, invariants and brute force on tiny inputs.
None of these tests reuses the oracle's own code for the expected value."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(12345)


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f32(x):
    return np.asarray(x, dtype=np.float32)


def _bf16_bits_torch(x32):
    return torch.from_numpy(np.ascontiguousarray(x32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# ----------------------------------------------------------------------------
# low-precision formats vs library conversions
# ----------------------------------------------------------------------------
def _pattern_sweep(n=1 << 20):
    bits = RNG.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
    specials = np.array([0, 0x80000000, 0x7F800000, 0xFF800000, 0x7F7FFFFF, 0x00000001, 0x00800000,
                         0x477FE000, 0x477FEFFF, 0x477FF000, 0x38800000, 0x33800000, 0x33000000, 0x33000001,
                         0x3F808000, 0x3F818000, 0x3F807FFF, 0x7F7F8000, 0x7F7FFFFF, 0x387FC000, 0x387FE000],
                        dtype=np.uint32)
    # every exponent with mantissas at and around the half-way points
    e = np.arange(256, dtype=np.uint32) << 23
    mids = np.concatenate([e | 0x1000, e | 0x3000, e | 0x0FFF, e | 0x1001, e | 0x8000, e | 0x18000, e | 0x7FFF])
    return np.concatenate([bits, specials, mids, mids | 0x80000000]).view(np.float32)


def test_narrow_f16_matches_numpy():
    x = _pattern_sweep()
    with np.errstate(over="ignore", invalid="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    got = oracle.narrow(x, "f16")
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all((got[nan] & 0x7C00) == 0x7C00) and np.all((got[nan] & 0x3FF) != 0)


def test_narrow_bf16_matches_torch():
    x = _pattern_sweep()
    ref = _bf16_bits_torch(x)
    got = oracle.narrow(x, "bf16")
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all((got[nan] & 0x7F80) == 0x7F80) and np.all((got[nan] & 0x7F) != 0)


def test_widen_matches_libraries():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f16 = h.view(np.float16).astype(np.float32)
    got = oracle.widen(h, "f16")
    nan = np.isnan(f16)
    assert np.array_equal(got[~nan].view(np.uint32), f16[~nan].view(np.uint32)) and np.all(np.isnan(got[nan]))
    bf = torch.from_numpy(h.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    got = oracle.widen(h, "bf16")
    nan = np.isnan(bf)
    assert np.array_equal(got[~nan].view(np.uint32), bf[~nan].view(np.uint32)) and np.all(np.isnan(got[nan]))


# ----------------------------------------------------------------------------
# accumulation
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_accumulate_first_is_plain_conversion(dt):
    x = (RNG.standard_normal(4096) * 1e-3).astype(np.float32)
    bits = x.astype(np.float16).view(np.uint16) if dt == "f16" else _bf16_bits_torch(x)
    acc = np.full(x.size, 123.0, np.float32)
    oracle.accumulate(acc, bits, dt, first=True)
    ref = bits.view(np.float16).astype(np.float32) if dt == "f16" else \
        torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    assert np.array_equal(acc.view(np.uint32), ref.view(np.uint32))


def test_accumulate_closed_form_integer_ramp():
    # g_k = k * 2^-10 for k = 1..a: every partial sum is exactly representable,
    # so the accumulator holds a(a+1)/2 * 2^-10 exactly.
    a = 37
    acc = np.zeros(256, np.float32)
    for k in range(1, a + 1):
        g = np.full(256, k * 2.0 ** -10, np.float16).view(np.uint16)
        oracle.accumulate(acc, g, "f16", first=(k == 1))
    assert np.all(acc == np.float32(a * (a + 1) / 2 * 2.0 ** -10))


def test_accumulate_brute_force_rationals():
    # each micro-step adds one binary16 value to the binary32 accumulator: the
    # stored value is the exact rational sum rounded once to binary32.
    a, n = 6, 64
    gs = [(RNG.standard_normal(n) * 10.0 ** RNG.integers(-6, 2)).astype(np.float16) for _ in range(a)]
    acc = np.zeros(n, np.float32)
    for k, g in enumerate(gs):
        oracle.accumulate(acc, g.view(np.uint16), "f16", first=(k == 0))
    for i in range(n):
        ref = Fraction(0)
        for k, g in enumerate(gs):
            exact = Fraction(float(g[i])) + (ref if k else 0)
            ref = Fraction(float(np.float32(float(exact))))  # one correctly rounded binary32 add
        assert float(acc[i]) == float(ref)


# ----------------------------------------------------------------------------
# replica reduction
# ----------------------------------------------------------------------------
def test_reduce_hand_derived_order_cases():
    for case in _golden("reduction_order.json")["cases"]:
        srcs = [np.array([v], np.float32) for v in case["replicas"]]
        got = oracle.reduce(srcs)
        assert float(got[0]) == case["gbar"], case


def test_reduce_single_replica_is_identity_and_pair_is_ieee_mean():
    x = (RNG.standard_normal(10000) * 1e-3).astype(np.float32)
    y = (RNG.standard_normal(10000) * 3e-2).astype(np.float32)
    assert np.array_equal(oracle.reduce([x]).view(np.uint32), x.view(np.uint32))
    ref = (x + y) / np.float32(2)  # numpy binary32 add, exact halving
    assert np.array_equal(oracle.reduce([x, y]).view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 7, 8, 16])
def test_reduce_identical_replicas_average_to_themselves(n):
    # n copies of small dyadic values: every partial sum is exact, so g_bar = x.
    x = (RNG.integers(-1000, 1000, 4096) * 2.0 ** -12).astype(np.float32)
    got = oracle.reduce([x] * n)
    assert np.array_equal(got, x)


def test_reduce_partials_widen_first():
    x = (RNG.standard_normal(4096) * 1e-2).astype(np.float32)
    parts = [_bf16_bits_torch(x * np.float32(r + 1)) for r in range(4)]
    wide = [oracle.widen(p, "bf16") for p in parts]
    assert np.array_equal(oracle.reduce(parts, "bf16"), oracle.reduce(wide, "f32"))


# ----------------------------------------------------------------------------
# statistics and per-step scalars
# ----------------------------------------------------------------------------
def test_stats_closed_form_constant_gradient():
    P = 1 << 20
    for c in (2.0 ** -10, -3.0, 0.0):
        ss, bad = oracle.stats(np.full(P, c, np.float32))
        assert bad == 0 and ss == c * c * P
        assert math.sqrt(ss) == abs(c) * 1024.0


def test_stats_against_fsum_and_nonfinite_count():
    x = (RNG.standard_normal(200003) * 1e-3).astype(np.float32)
    ss, bad = oracle.stats(x)
    ref = math.fsum(float(v) * float(v) for v in x.astype(np.float64))
    assert bad == 0 and abs(ss - ref) <= 1e-12 * ref
    y = x.copy()
    y[[0, 77, 200002]] = [np.inf, -np.inf, np.nan]
    assert oracle.stats(y)[1] == 3


def test_scaler_policy_matches_torch_amp_update():
    st = oracle.ScalarState(0.9, 0.999, "dynamic", 65536.0, 0.5, 2.0, 3)
    scale = torch.tensor([65536.0], dtype=torch.float32)
    tracker = torch.tensor([0], dtype=torch.int32)
    flags = [0, 0, 1, 0, 0, 0, 0, 1, 1, 0, 0, 0, 0, 0, 0, 0]
    for f in flags:
        rec = st.finalize(float("inf") if f else 1.0, 1 if f else 0, 0.0)
        torch._amp_update_scale_(scale, tracker, torch.tensor([float(f)]), 2.0, 0.5, 3)
        assert rec["scale"] == float(scale.item()) and rec["growth_tracker"] == int(tracker.item())
        assert rec["found_inf"] == f
    assert st.s.t == flags.count(0) and st.s.iter == len(flags)


def test_step_counter_and_bias_powers():
    st = oracle.ScalarState(0.9, 0.999)
    for t in range(1, 31):
        rec = st.finalize(1.0, 0, 0.0)
        assert rec["t"] == t
        assert abs(rec["beta1_pow"] - 0.9 ** t) <= 4 * t * 2.0 ** -53 * 0.9 ** t
        assert abs(rec["beta2_pow"] - 0.999 ** t) <= 4 * t * 2.0 ** -53 * 0.999 ** t
    st.finalize(0.0, 1, 0.0)  # skipped: t and the powers stay
    assert st.s.t == 30 and st.s.iter == 31


def test_clip_property():
    g = (RNG.standard_normal(100000) * 1e-2).astype(np.float32)
    ss, _ = oracle.stats(g)
    norm = math.sqrt(ss)
    st = oracle.ScalarState(0.9, 0.999, "static", 1024.0)
    rec = st.finalize(ss * 1024.0 ** 2, 0, 1.0)  # g carried a loss scale of 1024
    assert abs(rec["norm"] - norm) <= 1e-15 * norm
    if norm > 1.0:
        clipped = g.astype(np.float64) * 1024.0 * rec["gscale"]
        assert abs(np.linalg.norm(clipped) - 1.0) <= 1e-12
    st2 = oracle.ScalarState(0.9, 0.999)
    rec2 = st2.finalize(ss, 0, norm * 1.0001)
    assert rec2["clip"] == 1.0 and rec2["gscale"] == 1.0


# ----------------------------------------------------------------------------
# AdamW update
# ----------------------------------------------------------------------------
HP = dict(lr=1e-3, eps=1e-8, wd=0.01)


def _torch_adamw_step(w, m, v, g, t, lr, eps, wd, beta1=0.9, beta2=0.999):
    """One step of torch.optim.AdamW in binary64 from the given state."""
    p = torch.nn.Parameter(torch.from_numpy(w.astype(np.float64)))
    opt = torch.optim.AdamW([p], lr=lr, betas=(beta1, beta2), eps=eps, weight_decay=wd, foreach=False,
                            fused=False)
    p.grad = torch.from_numpy(g.astype(np.float64))
    opt.state[p] = {"step": torch.tensor(float(t - 1)), "exp_avg": torch.from_numpy(m.astype(np.float64)),
                    "exp_avg_sq": torch.from_numpy(v.astype(np.float64))}
    opt.step()
    s = opt.state[p]
    return p.detach().numpy(), s["exp_avg"].numpy(), s["exp_avg_sq"].numpy()


def _ulps(a, b):
    ai = a.view(np.int32).astype(np.int64)
    bi = b.view(np.int32).astype(np.int64)
    ai = np.where(ai < 0, -(ai & 0x7FFFFFFF), ai)
    bi = np.where(bi < 0, -(bi & 0x7FFFFFFF), bi)
    return np.abs(ai - bi)


def test_adamw_every_step_matches_torch_adamw_rounded():
    """Each oracle step equals torch.optim.AdamW (binary64) applied to the
    stored binary32 state and rounded to binary32; rounding-order differences
    in binary64 may move a value by one binary32 ulp at a near-tie."""
    n = 50000
    w = (RNG.standard_normal(n) * 0.02).astype(np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    p = oracle.narrow(w, "bf16")
    st = oracle.ScalarState(0.9, 0.999, "static", 1024.0)
    for t in range(1, 13):
        gbar = (RNG.standard_normal(n) * 1e-3 * 1024).astype(np.float32)
        ss, bad = oracle.stats(gbar)
        rec = st.finalize(ss, bad, 0.1)
        gtrue = gbar.astype(np.float64) * rec["gscale"]
        rw, rm, rv = _torch_adamw_step(w, m, v, gtrue, t, **HP)
        oracle.adamw(w, m, v, p, "bf16", gbar, st, **HP)
        for got, ref in ((w, rw), (m, rm), (v, rv)):
            d = _ulps(got, ref.astype(np.float32))
            assert d.max() <= 1 and np.count_nonzero(d) <= 5
        assert np.array_equal(p, _bf16_bits_torch(w))


def test_adamw_first_step_closed_form():
    """At t = 1 bias correction makes m_hat = g and v_hat = g^2, so
    w1 = w0 (1 - lr wd) - lr g / (|g| + eps) per element."""
    n = 20000
    w0 = (RNG.standard_normal(n) * 0.02).astype(np.float32)
    g = (RNG.standard_normal(n) * 1e-3).astype(np.float32)
    g[:10] = 0.0
    w, m, v = w0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    st = oracle.ScalarState(0.9, 0.999)
    st.finalize(*oracle.stats(g), 0.0)
    oracle.adamw(w, m, v, None, "bf16", g, st, **HP)
    gd = g.astype(np.float64)
    ref = (w0.astype(np.float64) * (1 - HP["lr"] * HP["wd"]) - HP["lr"] * gd / (np.abs(gd) + HP["eps"]))
    assert _ulps(w, ref.astype(np.float32)).max() <= 1
    assert np.array_equal(w[:10], (w0[:10].astype(np.float64) * (1 - 1e-5)).astype(np.float32))
    # |delta_adam| < lr always at t = 1
    step = w.astype(np.float64) - w0.astype(np.float64) * (1 - 1e-5)
    assert np.all(np.abs(step) < HP["lr"] * (1 + 1e-6))


def test_adamw_constant_gradient_closed_form():
    """With g_t = g every step and no weight decay the bias corrections cancel
    exactly in real arithmetic: every step moves w by -lr g / (|g| + eps)."""
    n, T = 4096, 25
    w0 = (RNG.standard_normal(n) * 0.02).astype(np.float32)
    g = (RNG.standard_normal(n) * 1e-3).astype(np.float32)
    w, m, v = w0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    st = oracle.ScalarState(0.9, 0.999)
    for _ in range(T):
        st.finalize(*oracle.stats(g), 0.0)
        oracle.adamw(w, m, v, None, "f16", g, st, lr=1e-3, eps=1e-8, wd=0.0)
    gd = g.astype(np.float64)
    ref = w0.astype(np.float64) - T * 1e-3 * gd / (np.abs(gd) + 1e-8)
    assert np.all(np.abs(w - ref) <= 1e-6 * np.abs(ref) + T * 2.0 ** -24 * 0.1)


def test_adamw_zero_gradient_is_pure_decay_and_skip_is_noop():
    n = 4096
    w0 = (RNG.standard_normal(n) * 0.02).astype(np.float32)
    w, m, v = w0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    st = oracle.ScalarState(0.9, 0.999)
    ref = w0.copy()
    for _ in range(7):
        st.finalize(0.0, 0, 0.0)
        oracle.adamw(w, m, v, None, "bf16", np.zeros(n, np.float32), st, **HP)
        ref = (ref.astype(np.float64) * (1 - HP["lr"] * HP["wd"])).astype(np.float32)
    assert np.array_equal(w, ref) and not m.any() and not v.any()
    before = [a.copy() for a in (w, m, v)]
    st.finalize(float("inf"), 1, 0.0)
    oracle.adamw(w, m, v, None, "bf16", np.full(n, np.inf, np.float32), st, **HP)
    for a, b in zip((w, m, v), before):
        assert np.array_equal(a, b)


def test_adamw_sharded_equals_unsharded():
    """Sharding changes the layout, not the update: the union of the updates
    of disjoint ranges equals one update of the whole range, bit for bit."""
    n = 100003
    w0 = (RNG.standard_normal(n) * 0.02).astype(np.float32)
    g = (RNG.standard_normal(n) * 1e-3).astype(np.float32)
    st = oracle.ScalarState(0.9, 0.999)
    st.finalize(*oracle.stats(g), 0.0)
    full = [w0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32), oracle.narrow(w0, "f16")]
    oracle.adamw(*full[:3], full[3], "f16", g, st, **HP)
    cuts = [0, 1, 12345, 50000, 50001, 99999, n]
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        part = [w0[lo:hi].copy(), np.zeros(hi - lo, np.float32), np.zeros(hi - lo, np.float32),
                np.zeros(hi - lo, np.uint16)]
        oracle.adamw(*part[:3], part[3], "f16", g[lo:hi].copy(), st, **HP)
        for a, b in zip(part, full):
            assert np.array_equal(a, b[lo:hi])


# ----------------------------------------------------------------------------
# the pages' printed figures and counting rules
# ----------------------------------------------------------------------------
def test_pages_figures():
    f = _golden("pages_figures.json")
    gb = f["global_batch_worked_example"]
    assert oracle.global_batch(gb["b"], gb["n"], gb["a"]) == gb["B_global"]
    d3 = f["global_batch_3d"]
    assert oracle.global_batch(4, d3["dp"], 8) == 8 * 4 * 8 != 64 * 4 * 8
    sb = f["state_bytes_per_param"]
    assert oracle.state_bytes(sb["params"]) == sb["total_bytes"]
    rng = f["state_bytes_range"]
    assert rng["lo"] <= oracle.state_bytes(1) <= rng["hi"]
    z3 = f["zero3_per_gpu"]
    assert oracle.state_bytes(z3["params"], z3["N"]) == z3["bytes"]
    ra = f["ring_allreduce_factor"]
    assert oracle.ring_allreduce_factor(ra["N"]) == ra["factor"]


# ----------------------------------------------------------------------------
# the whole-step driver
# ----------------------------------------------------------------------------
def _fns(w):
    def grad_fn(step, r, k, lo, hi, scale):
        return synth.grad_host(w, step, r, k, lo, hi, scale)

    def master_fn(lo, hi):
        return synth.master_host(w, lo, hi)

    return grad_fn, master_fn


def test_run_single_replica_single_microstep_is_conversion():
    w = workloads.tiny().with_(numel=(5000, 3), n=1, a=1, steps=1)
    gf, mf = _fns(w)
    res = oracle.run(w, 1, gf, mf, keep_gbar=(1,), threads=1, chunk=1000)
    ref = gf(1, 0, 1, 0, w.P, 1.0).view(np.float16).astype(np.float32)
    assert np.array_equal(res.gbar[1][(0, w.P)], ref)


def test_run_replicas_average_matches_definition_small():
    """n=3, a=2 on a ragged layout: g_bar equals the per-element definition
    written with exact rationals (each stored value rounded to binary32)."""
    w = workloads.tiny().with_(numel=(7, 1, 30), n=3, a=2, steps=1)
    gf, mf = _fns(w)
    res = oracle.run(w, 1, gf, mf, keep_gbar=(1,), threads=1, chunk=16)
    got = res.gbar[1][(0, w.P)]
    gs = {(r, k): gf(1, r, k, 0, w.P, 1.0).view(np.float16) for r in range(3) for k in (1, 2)}

    def r32(q):
        return Fraction(float(np.float32(float(q))))

    for i in range(w.P):
        acc = [r32(Fraction(float(gs[(r, 1)][i])) + Fraction(float(gs[(r, 2)][i]))) for r in range(3)]
        total = r32(acc[0] + acc[1]) + acc[2]
        assert float(got[i]) == float(r32(r32(total) / 3))


def test_skip_run_equals_clean_run_without_the_skipped_step():
    """Dynamic loss scale with an inf injected at step 3: the 5-step run equals
    a clean 4-step run on the inputs of steps 1, 2, 4, 5 (power-of-two scales
    cancel exactly), bit for bit."""
    base = workloads.zero3_rank_7b()
    P = 50000
    w = base.with_(numel=(P,), injections=((3, 0, 1, P // 2, float("inf")),))
    gf, mf = _fns(w)
    res = oracle.run(w, 5, gf, mf, threads=2, chunk=8192)
    assert [r["found_inf"] for r in res.scalars] == [0, 0, 1, 0, 0]
    assert [r["t"] for r in res.scalars] == [1, 2, 2, 3, 4]
    assert res.scalars[-1]["scale"] == 32768.0

    clean = w.with_(injections=())
    order = [1, 2, 4, 5]

    def gf2(step, r, k, lo, hi, scale):
        return synth.grad_host(clean, order[step - 1], r, k, lo, hi, scale)

    res2 = oracle.run(clean, 4, gf2, mf, threads=2, chunk=8192)
    for key in ("w", "m", "v", "p"):
        assert np.array_equal(res.state[(0, P)][key], res2.state[(0, P)][key])


def test_run_windows_equal_full_run():
    w = workloads.gpt2_small().with_(numel=(3000, 17, 4096, 5), n=2, a=3, steps=3, scaled_tensors=(1,))
    gf, mf = _fns(w)
    full = oracle.run(w, 3, gf, mf, threads=1, chunk=777)
    wins = [(0, 10), (2990, 3030), (7000, w.P)]
    part = oracle.run(w, 3, gf, mf, windows=wins, threads=3, chunk=777)
    for a, b in zip(full.scalars, part.scalars):
        assert a["norm"] == pytest.approx(b["norm"], rel=1e-14) and a["clip"] == pytest.approx(b["clip"], rel=1e-14)
    for lo, hi in wins:
        for key in ("w", "m", "v", "p"):
            assert np.array_equal(full.state[(0, w.P)][key][lo:hi], part.state[(lo, hi)][key])
