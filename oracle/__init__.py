"""CPU oracle of the data-parallel update step.

TEST INFRASTRUCTURE ONLY.  The tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg are the only code that imports this package; the
GPU library and its Python binding never do, and this package imports neither
of them.  Inputs come from the caller (the seeded generators in ``synth``).

What it computes (see ``oracle.c`` for the per-function citations):

1. accumulate each replica's ``a`` micro-step gradients into a binary32
   ``g_r`` ("Distributed Training: Split along the Four Axes ...", averaging
   formula paragraph and the b=4, a=8, n=8 worked example);
2. ``g_bar = (sum_r g_r) / n`` with one fixed pairwise order (same page,
   averaging formula and reduction-order paragraphs);
3. the global sum of squares and non-finite count of ``g_bar``;
4. per-step scalars: norm, clip factor, loss-scale bookkeeping, step count
   and bias-correction powers (loss scaling is training state: same page,
   checkpoint paragraph);
5. the AdamW update of the binary32 master, first and second moments on any
   range of the flat space, emitting the low-precision parameter ("Data vs
   Tensor vs Pipeline Parallelism", data parallelism section: 16 bytes per
   parameter; the ZeRO paragraph of the first page: a shard's update equals
   the unsharded one).

All arithmetic is binary64, rounded to binary32 exactly where the method stores
a value.  Accounting helpers (global batch, state bytes) restate the pages'
counting rules.
"""
from __future__ import annotations

import ctypes
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

DTYPES = {"f32": 0, "f16": 1, "bf16": 2}
SCALERS = {"none": 0, "static": 1, "dynamic": 2}


class Scalars(ctypes.Structure):
    _fields_ = [("t", ctypes.c_int64), ("iter", ctypes.c_int64), ("growth_tracker", ctypes.c_int64),
                ("beta1_pow", ctypes.c_double), ("beta2_pow", ctypes.c_double), ("scale", ctypes.c_double),
                ("found_inf", ctypes.c_int32), ("pad", ctypes.c_int32), ("sumsq", ctypes.c_double),
                ("norm", ctypes.c_double), ("clip", ctypes.c_double), ("gscale", ctypes.c_double)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_ if name != "pad"}


class Cfg(ctypes.Structure):
    _fields_ = [("beta1", ctypes.c_double), ("beta2", ctypes.c_double), ("scaler_mode", ctypes.c_int32),
                ("growth_interval", ctypes.c_int32), ("init_scale", ctypes.c_double),
                ("backoff", ctypes.c_double), ("growth", ctypes.c_double)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        L.oracle_widen.argtypes = [vp, i32, i64, vp]
        L.oracle_narrow.argtypes = [vp, i32, i64, vp]
        L.oracle_accumulate.argtypes = [vp, vp, i32, i64, i32]
        L.oracle_reduce.argtypes = [vp, ctypes.POINTER(vp), i32, i32, i64]
        L.oracle_stats.argtypes = [vp, i64, ctypes.POINTER(dbl), ctypes.POINTER(i64)]
        L.oracle_init.argtypes = [ctypes.POINTER(Scalars), ctypes.POINTER(Cfg)]
        L.oracle_finalize.argtypes = [ctypes.POINTER(Scalars), ctypes.POINTER(Cfg), dbl, i64, dbl]
        L.oracle_adamw.argtypes = [vp, vp, vp, vp, i32, vp, i64, ctypes.POINTER(Scalars), dbl, dbl, dbl, dbl, dbl]
        for f in ("oracle_widen", "oracle_narrow", "oracle_accumulate", "oracle_reduce", "oracle_stats",
                  "oracle_init", "oracle_finalize", "oracle_adamw"):
            getattr(L, f).restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags.c_contiguous
    return a.ctypes.data


# ----------------------------------------------------------------------------
# element-wise primitives
# ----------------------------------------------------------------------------
def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    """binary16 / bfloat16 bit patterns (uint16) to binary32 (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.size, dtype=np.float32)
    lib().oracle_widen(_ptr(bits), DTYPES[dtype], bits.size, _ptr(out))
    return out


def narrow(x: np.ndarray, dtype: str) -> np.ndarray:
    """binary32 to binary16 / bfloat16 bits, round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.size, dtype=np.uint16)
    lib().oracle_narrow(_ptr(x), DTYPES[dtype], x.size, _ptr(out))
    return out


def accumulate(acc: np.ndarray, g: np.ndarray, gdtype: str, first: bool) -> np.ndarray:
    """In place: ``acc = g`` on the first micro-step, else ``acc = acc + g``
    (binary32 storage)."""
    assert acc.dtype == np.float32 and acc.size == g.size
    g = np.ascontiguousarray(g)
    lib().oracle_accumulate(_ptr(acc), _ptr(g), DTYPES[gdtype], acc.size, int(bool(first)))
    return acc


def reduce(srcs: Sequence[np.ndarray], src_dtype: str = "f32") -> np.ndarray:
    """``(sum_r srcs[r]) / n`` in the fixed pairwise order, binary32 partial sums."""
    n = len(srcs)
    size = srcs[0].size
    arrs = [np.ascontiguousarray(s) for s in srcs]
    ptrs = (ctypes.c_void_p * n)(*[_ptr(s) for s in arrs])
    out = np.empty(size, dtype=np.float32)
    lib().oracle_reduce(_ptr(out), ptrs, DTYPES[src_dtype], n, size)
    return out


def stats(gbar: np.ndarray) -> Tuple[float, int]:
    gbar = np.ascontiguousarray(gbar, dtype=np.float32)
    s = ctypes.c_double()
    bad = ctypes.c_int64()
    lib().oracle_stats(_ptr(gbar), gbar.size, ctypes.byref(s), ctypes.byref(bad))
    return s.value, bad.value


class ScalarState:
    """The per-run scalar state (step count, bias-correction powers, loss
    scale, growth tracker) and the per-step derived values."""

    def __init__(self, beta1: float, beta2: float, scaler: str = "none", init_scale: float = 1.0,
                 backoff: float = 0.5, growth: float = 2.0, growth_interval: int = 2000):
        self.cfg = Cfg(beta1, beta2, SCALERS[scaler], growth_interval, init_scale, backoff, growth)
        self.s = Scalars()
        lib().oracle_init(ctypes.byref(self.s), ctypes.byref(self.cfg))

    def finalize(self, sumsq: float, nonfinite: int, max_norm: float) -> dict:
        lib().oracle_finalize(ctypes.byref(self.s), ctypes.byref(self.cfg), sumsq, nonfinite, max_norm)
        return self.s.as_dict()

    @property
    def scale(self) -> float:
        return self.s.scale


def adamw(w: np.ndarray, m: np.ndarray, v: np.ndarray, p: Optional[np.ndarray], pdtype: str,
          gbar: np.ndarray, st: ScalarState, lr: float, eps: float, wd: float) -> None:
    """In place on (w, m, v, p) over one range; no-op on a skipped step."""
    for a in (w, m, v, gbar):
        assert a.dtype == np.float32 and a.flags.c_contiguous and a.size == w.size
    pp = 0 if p is None else _ptr(p)
    lib().oracle_adamw(_ptr(w), _ptr(m), _ptr(v), pp, DTYPES[pdtype], _ptr(gbar), w.size, ctypes.byref(st.s),
                       lr, eps, wd, st.cfg.beta1, st.cfg.beta2)


# ----------------------------------------------------------------------------
# accounting, restating the pages' counting rules
# ----------------------------------------------------------------------------
def global_batch(b: int, n: int, a: int) -> int:
    """Samples per update: local micro-batch x data-parallel replicas x
    accumulation steps ("Distributed Training ...", averaging formula
    paragraph); tensor- and pipeline-parallel degrees do not enter (same page,
    3D-parallelism counting paragraph)."""
    return b * n * a


def state_bytes(params: int, shards: int = 1) -> float:
    """Model-state bytes per GPU at 16 bytes per parameter, divided over
    ``shards`` ZeRO-3 ranks ("Data vs Tensor vs Pipeline Parallelism", data
    parallelism section: 16 bytes per parameter and 16*Psi/N).  The 16 bytes
    read as 2 (low-precision parameter) + 2 (gradient) + 4 (binary32 master)
    + 4 + 4 (the two moments)."""
    return 16.0 * params / shards


def ring_allreduce_factor(N: int) -> float:
    """Bytes sent and received per GPU by a ring all-reduce, as a multiple of
    the gradient bytes (same section): 2 (N - 1) / N."""
    return 2.0 * (N - 1) / N


# ----------------------------------------------------------------------------
# the whole step, driven over a run of steps
# ----------------------------------------------------------------------------
GradFn = Callable[[int, int, int, int, int, float], np.ndarray]
MasterFn = Callable[[int, int], np.ndarray]


@dataclass
class RunResult:
    scalars: List[dict] = field(default_factory=list)            # per step, after finalize
    state: Dict[Tuple[int, int], Dict[str, np.ndarray]] = field(default_factory=dict)
    gbar: Dict[int, Dict[Tuple[int, int], np.ndarray]] = field(default_factory=dict)


def _step_chunk(w, step: int, lo: int, hi: int, scale: float, grad_fn: GradFn):
    """g_bar on [lo, hi) for one step: accumulation per replica, then the
    fixed-order reduction."""
    if w.partials:
        parts = [grad_fn(step, r, 1, lo, hi, scale) for r in range(w.n)]
        return reduce(parts, w.grad_dtype)
    accs = []
    for r in range(w.n):
        acc = np.empty(hi - lo, dtype=np.float32)
        for k in range(1, w.a + 1):
            accumulate(acc, grad_fn(step, r, k, lo, hi, scale), w.grad_dtype, first=(k == 1))
        accs.append(acc)
    return reduce(accs, "f32")


def run(w, steps: int, grad_fn: GradFn, master_fn: MasterFn, windows: Optional[Sequence[Tuple[int, int]]] = None,
        threads: int = 8, chunk: int = 1 << 20, keep_gbar: Sequence[int] = (),
        progress: Optional[Callable[[int, dict], None]] = None) -> RunResult:
    """Runs ``steps`` data-parallel steps of workload ``w`` and returns the
    state on ``windows`` (default: the whole flat range).

    The global statistics always cover the whole flat range [0, P); the
    update is applied on the windows only (each element's update depends on
    the global scalars and its own values alone).  ``progress(step,
    scalars)``, if given, is called after each step (reporting only)."""
    P = w.P
    windows = [(0, P)] if windows is None else [tuple(x) for x in windows]
    st = ScalarState(w.beta1, w.beta2, w.scaler, w.init_scale, w.backoff, w.growth, w.growth_interval)
    res = RunResult()
    for (lo, hi) in windows:
        m0 = np.ascontiguousarray(master_fn(lo, hi), dtype=np.float32).copy()
        res.state[(lo, hi)] = {"w": m0, "m": np.zeros(hi - lo, np.float32), "v": np.zeros(hi - lo, np.float32),
                               "p": narrow(m0, w.param_dtype)}
    bounds = [(c0, min(P, c0 + chunk)) for c0 in range(0, P, chunk)] if P else []

    for s in range(1, steps + 1):
        scale = st.scale

        def task(b):
            c0, c1 = b
            gbar = _step_chunk(w, s, c0, c1, scale, grad_fn)
            ss, bad = stats(gbar)
            kept = {}
            for (lo, hi) in windows:
                a0, a1 = max(lo, c0), min(hi, c1)
                if a0 < a1:
                    kept[(lo, hi, a0)] = gbar[a0 - c0:a1 - c0].copy()
            return ss, bad, kept

        if threads > 1 and len(bounds) > 1:
            with ThreadPoolExecutor(max_workers=threads) as ex:
                parts = list(ex.map(task, bounds))
        else:
            parts = [task(b) for b in bounds]
        sumsq = 0.0
        nonfinite = 0
        wgbar = {win: np.empty(win[1] - win[0], np.float32) for win in windows}
        for ss, bad, kept in parts:  # chunk order
            sumsq += ss
            nonfinite += bad
            for (lo, hi, a0), g in kept.items():
                wgbar[(lo, hi)][a0 - lo:a0 - lo + g.size] = g
        rec = st.finalize(sumsq, nonfinite, w.max_norm)
        res.scalars.append(rec)
        if s in keep_gbar:
            res.gbar[s] = {win: g.copy() for win, g in wgbar.items()}
        for win in windows:
            S = res.state[win]
            adamw(S["w"], S["m"], S["v"], S["p"], w.param_dtype, wgbar[win], st, w.lr, w.eps, w.weight_decay)
        if progress is not None:
            progress(s, rec)
    return res
