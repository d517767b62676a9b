"""Shared helpers of the GPU parity tests: run a workload through the HIP
library, run the same workload through the CPU oracle, compare.

Inputs on both sides come from the seeded generators in ``synth`` (device twin
on the GPU side, host twin on the oracle side); nothing the GPU computes is
fed to the oracle."""
from __future__ import annotations

import os
import sys
from typing import Dict, List, Tuple

import numpy as np
import torch

import oracle
import synth
from gradient_reduce_adam_amd import driver

THREADS = int(os.environ.get("DP_ORACLE_THREADS", str(min(16, len(os.sched_getaffinity(0))))))

# Tolerances stated for the step: binary32 master, m, v within 2e-6 relative
# with a 1e-9 absolute floor; the gradient norm within 1e-5 relative;
# low-precision parameters within 1 ulp; flags and counters exact.
RTOL_STATE = 2e-6
ATOL_STATE = 1e-9
RTOL_NORM = 1e-5
# Beyond the stated bars, the binary32 distance of master, m and v in ulp.
# Without clipping the library computes the update in binary64 in the
# oracle's order of operations, so the two must agree bit for bit.  With
# clipping the clip factor comes from the norm, whose summation order differs
# (within 1e-5), and a few ulp may follow; more than MAX_ULP_CLIPPED is a bug.
MAX_ULP_CLIPPED = 64


def ulp_bound(w) -> int:
    """The ulp bound of master, m and v for workload w: 0 without clipping,
    MAX_ULP_CLIPPED with it."""
    return 0 if w.max_norm == 0.0 else MAX_ULP_CLIPPED


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


# ----------------------------------------------------------------------------
# GPU side
# ----------------------------------------------------------------------------
class DeviceRun:
    """A workload on the GPU: the library's driver plus device-generated inputs."""

    def __init__(self, w, shards=None, chunk_elems: int = 0, fused: bool = True, single_pass: bool = False,
                 state_location: str = "hbm", stream=None, **extra):
        self.w = w
        self.d = driver.DPStep(w.numel, w.n, w.a, w.grad_dtype, w.param_dtype, lr=w.lr, eps=w.eps,
                               weight_decay=w.weight_decay, beta1=w.beta1, beta2=w.beta2, max_norm=w.max_norm,
                               scaler=w.scaler, init_scale=w.init_scale, backoff=w.backoff, growth=w.growth,
                               growth_interval=w.growth_interval, partials=w.partials, shards=shards,
                               chunk_elems=chunk_elems, fused=fused, single_pass=single_pass,
                               state_location=state_location, stream=stream, **extra)
        slots = w.n if (w.partials or fused) else 1  # the fused step holds every replica's gradient at once
        self.slots = [torch.empty(w.P, dtype=torch.int16, device="cuda") for _ in range(slots)]
        self.stream = self.d.stream.cuda_stream
        self.d.set_master(lambda ptr: synth.master_device(w, ptr, self.stream))
        self.states: List[dict] = []

    def produce(self, step: int, r: int, k: int, scale: float) -> int:
        buf = self.slots[r % len(self.slots)]
        synth.grad_device(self.w, step, r, k, buf.data_ptr(), scale, self.stream)
        return buf.data_ptr()

    def step(self) -> dict:
        s = self.d.step(self.produce, sync_scale=True)
        self.states.append(s)
        return s

    def run(self, steps: int) -> List[dict]:
        for _ in range(steps):
            self.step()
        return self.states

    def window(self, lo: int, hi: int) -> Dict[str, np.ndarray]:
        """master, m, v (of the current state bank), p and, when the run
        stores it, g_bar over [lo, hi)."""
        torch.cuda.synchronize()
        w_, m_, v_ = self.d.state_tensors()
        out = {"w": w_[lo:hi].cpu().numpy(), "m": m_[lo:hi].cpu().numpy(), "v": v_[lo:hi].cpu().numpy(),
               "p": self.d.param[lo:hi].view(torch.int16).cpu().numpy().view(np.uint16)}
        if self.d.gbar is not None:
            out["gbar"] = self.d.gbar[lo:hi].cpu().numpy()
        return out

    def close(self):
        self.d.close()
        del self.slots
        self.d = None
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


# ----------------------------------------------------------------------------
# oracle side
# ----------------------------------------------------------------------------
def oracle_run(w, steps: int, windows=None, keep_gbar=(), chunk: int = 1 << 20, progress=None):
    """The oracle's run of workload w; with clipping, each window's state also
    carries ``m_slack`` (see ``m_slack``)."""
    def grad_fn(step, r, k, lo, hi, scale):
        return synth.grad_host(w, step, r, k, lo, hi, scale)

    def master_fn(lo, hi):
        return synth.master_host(w, lo, hi)

    extra = set(range(1, steps + 1)) - set(keep_gbar) if w.max_norm > 0 else set()
    res = oracle.run(w, steps, grad_fn, master_fn, windows=windows, threads=THREADS, chunk=chunk,
                     keep_gbar=tuple(sorted(set(keep_gbar) | extra)), progress=progress)
    if w.max_norm > 0:
        for win, st in res.state.items():
            per_step = [(res.gbar[s][win], rec) for s, rec in enumerate(res.scalars, start=1)]
            st["m_slack"] = m_slack(w.P, w.beta1, per_step)
        for s in extra:
            res.gbar.pop(s, None)
    return res


def m_slack(P: int, beta1: float, steps) -> np.ndarray:
    """How far m may legitimately differ from the oracle's under clipping, per
    element, from the oracle's own per-step g_bar and scalars.

    The global norm is a binary64 sum of P non-negative squares whose order
    "Distributed Training: Split along the Four Axes of Data, Tensor, Pipeline,
    and State" leaves open (its reduction-order paragraph).  Two orders agree
    to (P - 1) * 2^-53 relative (the recursive-summation bound), so the clip
    factor and every g = g_bar * gscale may differ by delta = (P + 8) * 2^-53
    relative (a few more roundings in the square root and the division).
    Each step's m, stored in binary32, may then round to a neighbouring value:
    one ulp, at most 2^-23 * max|g| since |m_s| <= max_{r<=s} |g_r|.  Both
    carry over with weight beta1 per step, so
        |dm_t| <= sum_s beta1^(t-s) * ((1 - beta1) * delta * |g_s| + ulp(m_s))
               <= (delta + 2^-23 / (1 - beta1)) * max_s |g_s|.
    Where m nearly cancels, this exceeds 64 binary32 ulp of m itself; w and v
    have no such cancellation.  Skipped steps (found_inf) do not touch m."""
    delta = (P + 8) * 2.0 ** -53
    bound = (delta + 2.0 ** -23 / (1.0 - beta1)) * 1.01
    gmax = None
    for gbar, rec in steps:
        if gmax is None:
            gmax = np.zeros(gbar.size, np.float64)
        if rec["found_inf"]:
            continue
        np.maximum(gmax, np.abs(gbar.astype(np.float64) * rec["gscale"]), out=gmax)
    return bound * gmax if gmax is not None else np.zeros(0, np.float64)


# ----------------------------------------------------------------------------
# comparison
# ----------------------------------------------------------------------------
def ulps32(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    ai = a.view(np.int32).astype(np.int64)
    bi = b.view(np.int32).astype(np.int64)
    ai = np.where(ai < 0, -(ai & 0x7FFFFFFF), ai)
    bi = np.where(bi < 0, -(bi & 0x7FFFFFFF), bi)
    return np.abs(ai - bi)


def ulps16(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    ai = a.astype(np.int64)
    bi = b.astype(np.int64)
    ai = np.where(ai >= 0x8000, -(ai & 0x7FFF), ai)
    bi = np.where(bi >= 0x8000, -(bi & 0x7FFF), bi)
    return np.abs(ai - bi)


def assert_state_close(got: Dict[str, np.ndarray], ref: Dict[str, np.ndarray], max_ulp: int,
                       where: str = "") -> dict:
    """master, m and v within the stated tolerance and within max_ulp binary32
    ulp of the oracle (finite pairs; a non-finite value must match its own
    kind); the low-precision parameters within 1 ulp.  Under clipping an
    element of m beyond max_ulp passes if it lies within ``ref["m_slack"]``,
    the difference the norm's summation order allows.  Returns the largest
    ulp distance of each."""
    report = {}
    for key in ("w", "m", "v"):
        g, r = got[key], ref[key]
        assert g.shape == r.shape, (key, g.shape, r.shape)
        gf, rf = g.astype(np.float64), r.astype(np.float64)
        # a non-finite value matches only its own kind: NaN for NaN, an
        # infinity for the infinity of the same sign
        fin = np.isfinite(gf) & np.isfinite(rf)
        same_kind = (np.isnan(gf) & np.isnan(rf)) | (gf == rf)
        odd = np.flatnonzero(~fin & ~same_kind)
        assert odd.size == 0, f"{where} {key}: {odd.size} non-finite mismatches, first at {odd[:5]}: " \
                              f"gpu {g[odd[:5]]} oracle {r[odd[:5]]}"
        err = np.where(fin, np.abs(np.where(fin, gf, 0.0) - np.where(fin, rf, 0.0)), 0.0)
        lim = RTOL_STATE * np.abs(np.where(fin, rf, 0.0)) + ATOL_STATE
        bad = np.flatnonzero(err > lim)
        assert bad.size == 0, f"{where} {key}: {bad.size} elements out of tolerance, first at {bad[:5]}: " \
                              f"gpu {g[bad[:5]]} oracle {r[bad[:5]]}"
        u = np.where(fin, ulps32(g, r), 0)
        report[key + "_max_ulp"] = int(u.max()) if g.size else 0
        far_mask = u > max_ulp
        if key == "m" and "m_slack" in ref:  # clipping: the norm's summation order (see m_slack)
            within = far_mask & (err <= ref["m_slack"])
            report["m_within_norm_order_slack"] = int(np.count_nonzero(within))
            far_mask &= ~within
        far = np.flatnonzero(far_mask)
        assert far.size == 0, f"{where} {key}: {far.size} elements more than {max_ulp} ulp from the oracle " \
                              f"(max {report[key + '_max_ulp']}), first at {far[:5]}: gpu {g[far[:5]]} " \
                              f"oracle {r[far[:5]]}"
    pu = ulps16(got["p"], ref["p"])
    report["p_max_ulp"] = int(pu.max()) if pu.size else 0
    assert report["p_max_ulp"] <= 1, f"{where} params differ by {report['p_max_ulp']} ulp"
    return report


def assert_scalars_match(gpu: dict, ref: dict, where: str = "") -> None:
    for k in ("t", "iter", "found_inf", "growth_tracker", "scale"):
        assert gpu[k] == ref[k], f"{where} {k}: gpu {gpu[k]} oracle {ref[k]}"
    for k in ("beta1_pow", "beta2_pow"):
        assert gpu[k] == ref[k], f"{where} {k}: gpu {gpu[k]!r} oracle {ref[k]!r}"
    if np.isfinite(ref["norm"]):
        assert abs(gpu["norm"] - ref["norm"]) <= RTOL_NORM * abs(ref["norm"]), (where, gpu["norm"], ref["norm"])
        assert abs(gpu["clip"] - ref["clip"]) <= RTOL_NORM * abs(ref["clip"]), (where, gpu["clip"], ref["clip"])
    else:
        assert not np.isfinite(gpu["norm"])


def sample_windows(w, count: int = 24, width: int = 4096, seed: int = 0, edge: int = 128) -> List[Tuple[int, int]]:
    """First and last elements, a window of +-edge elements around every
    tensor boundary, windows straddling chunk boundaries, around each injected
    element, and seeded random ones."""
    P = w.P
    rng = np.random.default_rng(seed)
    wins = [(0, min(P, width)), (max(0, P - width), P)]
    off = w.offsets
    for t in range(1, w.T):
        c = int(off[t])
        wins.append((max(0, c - edge), min(P, c + edge)))
    for c in (65536, 3 * 65536, P // 2 // 65536 * 65536):
        if 0 < c < P:
            wins.append((max(0, c - 64), min(P, c + 64)))
    for (_, _, _, idx, _) in w.injections:
        wins.append((max(0, idx - 256), min(P, idx + 256)))
    for _ in range(count):
        lo = int(rng.integers(0, max(1, P - width)))
        wins.append((lo, min(P, lo + width)))
    wins = sorted(set(wins))
    merged: List[Tuple[int, int]] = []
    for lo, hi in wins:
        if merged and lo <= merged[-1][1]:
            merged[-1] = (merged[-1][0], max(hi, merged[-1][1]))
        else:
            merged.append((lo, hi))
    return merged
