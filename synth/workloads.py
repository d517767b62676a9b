"""The five workloads of the data-parallel update step, with their seeded
input recipes.

Shapes and hyperparameters are the benchmark configurations; everything not
stated there follows the readings recorded in the design notes (hyperparameters
of the tiny step reused everywhere, parameter dtype equal to the gradient dtype
unless stated, gradients stored already multiplied by the loss scale).

Input recipe, for every workload:

* master weights: stream ``(seed, MASTER, 0, 0, 0)``, position = flat index,
  standard deviation ``master_sigma``, binary32;
* gradient of replica ``r`` at micro-step ``k`` of step ``s`` (all 1-based for
  ``s`` and ``k``): stream ``(seed, GRAD, s, r, k)``, position = flat index,
  standard deviation ``grad_sigma`` (times ``grad_multiplier`` on the tensors
  in ``scaled_tensors``), times the loss scale, rounded into ``grad_dtype``;
* an injected non-finite value, where a workload asks for one, overwrites one
  element of one replica's gradient after generation.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    numel: Tuple[int, ...]
    n: int                      # data-parallel replicas held in this GPU's memory
    a: int                      # micro-steps accumulated per update
    grad_dtype: str             # 'f16' | 'bf16'
    param_dtype: str            # 'f16' | 'bf16'
    steps: int
    grad_sigma: float
    master_sigma: float = 0.02
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    max_norm: float = 0.0       # global-norm clip threshold; 0 disables clipping
    scaler: str = "none"        # 'none' | 'static' | 'dynamic'
    init_scale: float = 1.0
    backoff: float = 0.5
    growth: float = 2.0
    growth_interval: int = 2000
    partials: bool = False      # gradients arrive as n low-precision partials (a == 1)
    scaled_tensors: Tuple[int, ...] = ()
    grad_multiplier: float = 100.0
    # injected non-finite gradient values: (step, replica, micro, flat index, value)
    injections: Tuple[Tuple[int, int, int, int, float], ...] = ()

    @property
    def P(self) -> int:
        return int(sum(self.numel))

    @property
    def T(self) -> int:
        return len(self.numel)

    @property
    def offsets(self) -> np.ndarray:
        off = np.zeros(self.T + 1, dtype=np.int64)
        np.cumsum(np.asarray(self.numel, dtype=np.int64), out=off[1:])
        return off

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# ----------------------------------------------------------------------------
# layouts
# ----------------------------------------------------------------------------
def gpt2_small_layout() -> Tuple[int, ...]:
    """GPT-2-small parameter tensors in model order: token and position
    embeddings, 12 blocks of (ln_1 w/b, qkv w/b, attn proj w/b, ln_2 w/b,
    fc w/b, mlp proj w/b), final norm w/b.  148 tensors, 124,439,808 params."""
    d, v, ctx = 768, 50257, 1024
    t: List[int] = [v * d, ctx * d]
    for _ in range(12):
        t += [d, d, d * 3 * d, 3 * d, d * d, d, d, d, d * 4 * d, 4 * d, 4 * d * d, d]
    t += [d, d]
    return tuple(t)


def llama7b_layout() -> Tuple[int, ...]:
    """The 7B layout named by the workload: a 32000x4096 embedding followed by
    32 layers of four 4096x4096 and three 4096x11008 matrices.  225 tensors,
    6,607,077,376 params."""
    h, f = 4096, 11008
    t: List[int] = [32000 * h]
    for _ in range(32):
        t += [h * h] * 4 + [h * f] * 3
    return tuple(t)


def select_scaled_tensors(seed: int, T: int, fraction: float = 0.01) -> Tuple[int, ...]:
    """ceil(fraction * T) tensor indices, chosen by the seeded hash rank of the
    tensor index (smallest hashes win), returned sorted."""
    from . import ROLE_SELECT, hash_at, stream_key
    k = int(np.ceil(fraction * T - 1e-12))
    key = stream_key(seed, ROLE_SELECT, 0, 0, 0)
    ranked = sorted(range(T), key=lambda i: hash_at(key, i))
    return tuple(sorted(ranked[:k]))


# ----------------------------------------------------------------------------
# the five workloads
# ----------------------------------------------------------------------------
def tiny() -> Workload:
    """1,048,576 params in one tensor, n=4, a=2, fp16 gradients N(0, 1e-3),
    AdamW lr 1e-3, betas (0.9, 0.999), eps 1e-8, wd 0.01, no clipping, 10
    steps, unsharded."""
    return Workload(name="tiny", seed=1, numel=(1 << 20,), n=4, a=2, grad_dtype="f16", param_dtype="f16",
                    steps=10, grad_sigma=1e-3)


def gpt2_small() -> Workload:
    """GPT-2-small ragged layout (148 tensors), bf16 gradients N(0, 1e-3) with
    1% of tensors scaled x100, n=8, a=8 (b=4 gives a global batch of 256),
    global-norm clip 1.0, 20 steps."""
    numel = gpt2_small_layout()
    return Workload(name="gpt2_small", seed=2, numel=numel, n=8, a=8, grad_dtype="bf16", param_dtype="bf16",
                    steps=20, grad_sigma=1e-3, max_norm=1.0,
                    scaled_tensors=select_scaled_tensors(2, len(numel)))


def zero3_rank_7b() -> Workload:
    """One rank's ZeRO-3 share of a 7e9-param model over N=8: an 875M-param
    flat shard; 8 incoming bf16 gradient partials N(0, 1e-4) reduced then
    applied; a=1; dynamic loss scale 65536 with one +inf injected at step 3
    (replica 0, middle element); 5 steps."""
    P = 7_000_000_000 // 8
    return Workload(name="zero3_rank_7b", seed=3, numel=(P,), n=8, a=1, grad_dtype="bf16", param_dtype="bf16",
                    steps=5, grad_sigma=1e-4, scaler="dynamic", init_scale=65536.0, partials=True,
                    injections=((3, 0, 1, P // 2, float("inf")),))


def unsharded_7b() -> Workload:
    """The 7B layout unsharded on one GPU: n=1, a=8 micro-steps of bf16
    gradients N(0, 1e-4), fp32 accumulator, 3 steps."""
    return Workload(name="unsharded_7b", seed=4, numel=llama7b_layout(), n=1, a=8, grad_dtype="bf16",
                    param_dtype="bf16", steps=3, grad_sigma=1e-4)


def tp_column_slice() -> Workload:
    """The t=8 column slice 131072x32768 of the 131072x262144 MLP weight
    (2^32 params): fp16 params and gradients N(0, 1e-4) under a static loss
    scale of 1024, n=4, a=4, global-norm clip 1.0, 3 steps."""
    return Workload(name="tp_column_slice", seed=5, numel=(131072 * 32768,), n=4, a=4, grad_dtype="f16",
                    param_dtype="f16", steps=3, grad_sigma=1e-4, max_norm=1.0, scaler="static",
                    init_scale=1024.0)


BY_INDEX = (tiny, gpt2_small, zero3_rank_7b, unsharded_7b, tp_column_slice)


def by_name(name: str) -> Workload:
    for f in BY_INDEX:
        if f.__name__ == name:
            return f()
    raise KeyError(name)


# ----------------------------------------------------------------------------
# segments of the flat space with their generator constants
# ----------------------------------------------------------------------------
def grad_segments(w: Workload, lo: int, hi: int, loss_scale: float):
    """Yields (flat_start, count, c) pieces of [lo, hi) with the generator
    constant of each piece: a value depends only on its stream position and
    its tensor's constant, so runs of tensors that share a constant are one
    piece (one generator launch)."""
    from . import scale_constant
    off = w.offsets
    scaled = set(w.scaled_tensors)
    t = int(np.searchsorted(off, lo, side="right") - 1)
    pos = lo
    run_start, run_c = lo, None
    while pos < hi:
        end = min(hi, int(off[t + 1]))
        if end > pos:
            mult = w.grad_multiplier if t in scaled else 1.0
            c = scale_constant(w.grad_sigma, mult, loss_scale)
            if run_c is not None and c != run_c:
                yield run_start, pos - run_start, run_c
                run_start = pos
            run_c = c
        pos = end
        t += 1
    if run_c is not None and hi > run_start:
        yield run_start, hi - run_start, run_c
