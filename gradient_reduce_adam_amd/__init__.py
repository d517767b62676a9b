"""Python binding of ``libdpstep.so``, the gfx950 library of the data-parallel
gradient reduce + AdamW step.

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  The functions keep the C names (``dp_plan_create``,
``dp_accumulate``, ``dp_reduce_replicas``, ``dp_grad_stats``,
``dp_adam_step``, ...) and raise :class:`DpError` on a non-zero status;
:class:`Plan` wraps one plan.  Buffers are passed as device addresses (ints) or
as objects with ``data_ptr()`` (torch tensors); streams as ``hipStream_t``
handles (ints) or ``None`` for torch's current stream.  There is no CPU
fallback: importing this package fails if the library is not built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Iterable, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdpstep.so")

# enums of dpstep.h
(DP_OK, DP_ERR_INVALID_ARG, DP_ERR_BAD_LAYOUT, DP_ERR_UNBOUND, DP_ERR_RANGE, DP_ERR_STATE, DP_ERR_OOM, DP_ERR_HIP,
 DP_ERR_IO, DP_ERR_CORRUPT) = range(10)
DP_F32, DP_F16, DP_BF16 = 0, 1, 2
(DP_ROLE_PARAM, DP_ROLE_MASTER, DP_ROLE_EXP_AVG, DP_ROLE_EXP_AVG_SQ, DP_ROLE_GRAD, DP_ROLE_ACC,
 DP_ROLE_GBAR) = range(7)
DP_SCALER_NONE, DP_SCALER_STATIC, DP_SCALER_DYNAMIC = 0, 1, 2
DP_MAX_REPLICAS = 16
DP_DEFAULT_CHUNK = 16384
DP_STATIC_MAX_PARAMS = 1 << 30
DP_STATIC_SCRATCH_BYTES = 51920896

DTYPES = {"f32": DP_F32, "f16": DP_F16, "bf16": DP_BF16}
SCALERS = {"none": DP_SCALER_NONE, "static": DP_SCALER_STATIC, "dynamic": DP_SCALER_DYNAMIC}
ROLES = {"param": DP_ROLE_PARAM, "master": DP_ROLE_MASTER, "exp_avg": DP_ROLE_EXP_AVG,
         "exp_avg_sq": DP_ROLE_EXP_AVG_SQ, "grad": DP_ROLE_GRAD, "acc": DP_ROLE_ACC, "gbar": DP_ROLE_GBAR}

# every exported symbol of dpstep.h
EXPORTS = ("dp_abi_version", "dp_status_string", "dp_last_error", "dp_plan_create", "dp_plan_destroy",
           "dp_plan_info_get", "dp_plan_chunks", "dp_plan_bind_flat", "dp_plan_bind_tensors",
           "dp_plan_prepare_range", "dp_plan_drop_ranges", "dp_state_init", "dp_accumulate", "dp_accumulate_all",
           "dp_accumulate_all_range", "dp_accumulate_reduce", "dp_accumulate_reduce_range",
           "dp_reduce_replicas", "dp_reduce_replicas_range", "dp_grad_stats", "dp_adam_step", "dp_reduce_adam_step", "dp_reduce_adam_step_noalloc", "dp_reduce_adam_range",
           "dp_reduce_adam_finish", "dp_read_state",
           "dp_ckpt_write_shard", "dp_ckpt_commit", "dp_ckpt_read", "dp_checkpoint_save", "dp_checkpoint_commit",
           "dp_checkpoint_load")


class Layout(ctypes.Structure):
    _fields_ = [("num_tensors", ctypes.c_int32), ("n_replicas", ctypes.c_int32),
                ("numel", ctypes.POINTER(ctypes.c_int64)), ("grad_dtype", ctypes.c_int),
                ("param_dtype", ctypes.c_int), ("chunk_elems", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class StateCfg(ctypes.Structure):
    _fields_ = [("beta1", ctypes.c_double), ("beta2", ctypes.c_double), ("scaler_mode", ctypes.c_int32),
                ("growth_interval", ctypes.c_int32), ("init_scale", ctypes.c_double),
                ("backoff", ctypes.c_double), ("growth", ctypes.c_double)]


class AdamHparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double)]


class StepState(ctypes.Structure):
    _fields_ = [("t", ctypes.c_int64), ("iter", ctypes.c_int64), ("growth_tracker", ctypes.c_int64),
                ("beta1_pow", ctypes.c_double), ("beta2_pow", ctypes.c_double), ("scale", ctypes.c_double),
                ("found_inf", ctypes.c_int32), ("bank", ctypes.c_int32), ("sumsq", ctypes.c_double),
                ("norm", ctypes.c_double), ("clip", ctypes.c_double), ("gscale", ctypes.c_double)]

    def as_dict(self) -> dict:
        return {k: getattr(self, k) for k, _ in self._fields_ if k != "reserved"}


class PlanInfo(ctypes.Structure):
    _fields_ = [("params", ctypes.c_int64), ("num_chunks", ctypes.c_int64), ("num_tensors", ctypes.c_int32),
                ("n_replicas", ctypes.c_int32), ("chunk_elems", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("state_bytes", ctypes.c_double), ("bytes_accumulate_first", ctypes.c_double),
                ("bytes_accumulate", ctypes.c_double), ("bytes_reduce_acc", ctypes.c_double),
                ("bytes_reduce_partials", ctypes.c_double), ("bytes_accumulate_reduce", ctypes.c_double),
                ("bytes_stats_scan", ctypes.c_double),
                ("bytes_adam", ctypes.c_double), ("bytes_reduce_adam", ctypes.c_double),
                ("bytes_reduce_adam_partials", ctypes.c_double)]

    def as_dict(self) -> dict:
        return {k: getattr(self, k) for k, _ in self._fields_ if k != "reserved"}


class Chunk(ctypes.Structure):
    _fields_ = [("flat", ctypes.c_int64), ("offset", ctypes.c_int64), ("tensor", ctypes.c_int32),
                ("len", ctypes.c_int32)]


CHUNK_DTYPE = np.dtype([("flat", np.int64), ("offset", np.int64), ("tensor", np.int32), ("len", np.int32)])


class DpError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


_STATUS_NAMES = dict(enumerate(("DP_OK", "DP_ERR_INVALID_ARG", "DP_ERR_BAD_LAYOUT", "DP_ERR_UNBOUND", "DP_ERR_RANGE",
                                 "DP_ERR_STATE", "DP_ERR_OOM", "DP_ERR_HIP", "DP_ERR_IO", "DP_ERR_CORRUPT")))


def _hip_runtimes() -> set:
    try:
        with open("/proc/self/maps") as f:
            return {ln.split()[-1] for ln in f if "libamdhip64" in ln}
    except OSError:
        return set()


def _load():
    # The library must share the HIP runtime of whoever owns the device memory
    # and streams it is handed.  torch ships its own runtime; importing torch
    # first makes the loader resolve the library's libamdhip64.so.7 to that
    # already-loaded copy instead of mapping a second runtime.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built (run __graft_entry__.build()); "
                          "the HIP library is required, there is no fallback")
    L = ctypes.CDLL(LIB_PATH)
    runtimes = _hip_runtimes()
    if len(runtimes) > 1:
        raise ImportError("two HIP runtimes are mapped into this process (" + ", ".join(sorted(runtimes)) +
                          "); import torch before loading libdpstep.so so both use one runtime")
    vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    PP = ctypes.POINTER(vp)
    sig = {
        "dp_abi_version": (ctypes.c_int, []),
        "dp_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "dp_last_error": (ctypes.c_char_p, []),
        "dp_plan_create": (ctypes.c_int, [ctypes.POINTER(Layout), PP]),
        "dp_plan_destroy": (ctypes.c_int, [vp]),
        "dp_plan_info_get": (ctypes.c_int, [vp, ctypes.POINTER(PlanInfo)]),
        "dp_plan_chunks": (ctypes.c_int, [vp, i64, i64, i64, i64, vp, ctypes.POINTER(i64)]),
        "dp_plan_bind_flat": (ctypes.c_int, [vp, ctypes.c_int, i32, vp]),
        "dp_plan_bind_tensors": (ctypes.c_int, [vp, ctypes.c_int, i32, PP]),
        "dp_plan_prepare_range": (ctypes.c_int, [vp, i64, i64]),
        "dp_plan_drop_ranges": (ctypes.c_int, [vp]),
        "dp_state_init": (ctypes.c_int, [vp, ctypes.POINTER(StateCfg), vp]),
        "dp_accumulate": (ctypes.c_int, [vp, i32, i32, i32, vp]),
        "dp_accumulate_all": (ctypes.c_int, [vp, i32, vp]),
        "dp_accumulate_all_range": (ctypes.c_int, [vp, i32, i64, i64, vp]),
        "dp_accumulate_reduce": (ctypes.c_int, [vp, vp]),
        "dp_accumulate_reduce_range": (ctypes.c_int, [vp, i64, i64, vp]),
        "dp_reduce_replicas": (ctypes.c_int, [vp, ctypes.c_int, vp]),
        "dp_reduce_replicas_range": (ctypes.c_int, [vp, ctypes.c_int, i64, i64, vp]),
        "dp_grad_stats": (ctypes.c_int, [vp, i32, dbl, vp]),
        "dp_adam_step": (ctypes.c_int, [vp, ctypes.POINTER(AdamHparams), i64, i64, vp]),
        "dp_reduce_adam_step": (ctypes.c_int, [vp, ctypes.POINTER(AdamHparams), vp]),
        "dp_reduce_adam_step_noalloc": (ctypes.c_int, [i64, i32, ctypes.c_int, ctypes.c_int, PP, PP, PP, PP, PP, vp,
                                                       vp, ctypes.POINTER(StateCfg), ctypes.POINTER(AdamHparams),
                                                       vp]),
        "dp_reduce_adam_range": (ctypes.c_int, [vp, ctypes.POINTER(AdamHparams), i64, i64, vp]),
        "dp_reduce_adam_finish": (ctypes.c_int, [vp, vp]),
        "dp_read_state": (ctypes.c_int, [vp, ctypes.POINTER(StepState), vp]),
        "dp_ckpt_write_shard": (ctypes.c_int, [ctypes.c_char_p, i64, ctypes.POINTER(Layout), i64, i64, vp, vp, vp,
                                               vp]),
        "dp_ckpt_commit": (ctypes.c_int, [ctypes.c_char_p, i64, ctypes.POINTER(Layout), ctypes.POINTER(StepState),
                                          ctypes.POINTER(StateCfg)]),
        "dp_ckpt_read": (ctypes.c_int, [ctypes.c_char_p, ctypes.POINTER(Layout), i64, i64, vp, vp, vp, vp,
                                        ctypes.POINTER(StepState), ctypes.POINTER(StateCfg), ctypes.POINTER(i64)]),
        "dp_checkpoint_save": (ctypes.c_int, [vp, ctypes.c_char_p, i64, i64, i64, vp]),
        "dp_checkpoint_commit": (ctypes.c_int, [vp, ctypes.c_char_p, i64, vp]),
        "dp_checkpoint_load": (ctypes.c_int, [vp, ctypes.c_char_p, i64, i64, i32, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return L


lib = _load()


def _check(status: int) -> None:
    if status != DP_OK:
        raise DpError(status, lib.dp_last_error().decode(errors="replace"))


def _addr(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(s) -> int:
    if s is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(s, int):
        return s
    return int(s.cuda_stream)


# ----------------------------------------------------------------------------
# the C entry points, one to one
# ----------------------------------------------------------------------------
def dp_abi_version() -> int:
    return int(lib.dp_abi_version())


def dp_status_string(status: int) -> str:
    return lib.dp_status_string(status).decode()


def dp_last_error() -> str:
    return lib.dp_last_error().decode(errors="replace")


def dp_plan_create(numel: Sequence[int], n_replicas: int, grad_dtype: str, param_dtype: str,
                   chunk_elems: int = 0) -> int:
    arr = (ctypes.c_int64 * max(len(numel), 1))(*[int(x) for x in numel])
    lay = Layout(len(numel), int(n_replicas), arr, DTYPES[grad_dtype], DTYPES[param_dtype], int(chunk_elems), 0)
    out = ctypes.c_void_p()
    _check(lib.dp_plan_create(ctypes.byref(lay), ctypes.byref(out)))
    return int(out.value)


def dp_plan_destroy(plan: int) -> None:
    _check(lib.dp_plan_destroy(ctypes.c_void_p(plan)))


def dp_plan_info_get(plan: int) -> dict:
    info = PlanInfo()
    _check(lib.dp_plan_info_get(ctypes.c_void_p(plan), ctypes.byref(info)))
    return info.as_dict()


def dp_plan_chunks(plan: int, begin: int, end: int) -> np.ndarray:
    count = ctypes.c_int64()
    _check(lib.dp_plan_chunks(ctypes.c_void_p(plan), begin, end, 0, 0, None, ctypes.byref(count)))
    out = np.zeros(count.value, dtype=CHUNK_DTYPE)
    if count.value:
        _check(lib.dp_plan_chunks(ctypes.c_void_p(plan), begin, end, 0, count.value, out.ctypes.data,
                                  ctypes.byref(count)))
    return out


def dp_plan_bind_flat(plan: int, role: int, replica: int, base) -> None:
    _check(lib.dp_plan_bind_flat(ctypes.c_void_p(plan), role, replica, ctypes.c_void_p(_addr(base))))


def dp_plan_bind_tensors(plan: int, role: int, replica: int, ptrs: Iterable,
                         num_tensors: Optional[int] = None) -> None:
    """The library reads exactly one pointer per tensor of the plan, so the
    list's length is checked first (num_tensors: the plan's, if known)."""
    ptrs = [_addr(p) for p in ptrs]
    if num_tensors is None:
        num_tensors = dp_plan_info_get(plan)["num_tensors"]
    if len(ptrs) != num_tensors:
        raise ValueError(f"bind_tensors: {len(ptrs)} pointers for a plan of {num_tensors} tensors")
    arr = (ctypes.c_void_p * max(len(ptrs), 1))(*ptrs)
    _check(lib.dp_plan_bind_tensors(ctypes.c_void_p(plan), role, replica, arr))


def dp_plan_prepare_range(plan: int, begin: int, end: int) -> None:
    _check(lib.dp_plan_prepare_range(ctypes.c_void_p(plan), begin, end))


def dp_plan_drop_ranges(plan: int) -> None:
    _check(lib.dp_plan_drop_ranges(ctypes.c_void_p(plan)))


def dp_state_init(plan: int, beta1: float, beta2: float, scaler: str = "none", init_scale: float = 1.0,
                  backoff: float = 0.5, growth: float = 2.0, growth_interval: int = 2000, stream=None) -> None:
    cfg = StateCfg(beta1, beta2, SCALERS[scaler], growth_interval, init_scale, backoff, growth)
    _check(lib.dp_state_init(ctypes.c_void_p(plan), ctypes.byref(cfg), ctypes.c_void_p(_stream(stream))))


def dp_accumulate(plan: int, replica: int, first: bool, emit_stats: bool = False, stream=None) -> None:
    _check(lib.dp_accumulate(ctypes.c_void_p(plan), replica, int(bool(first)), int(bool(emit_stats)),
                             ctypes.c_void_p(_stream(stream))))


def dp_accumulate_all(plan: int, first: bool, stream=None) -> None:
    _check(lib.dp_accumulate_all(ctypes.c_void_p(plan), int(bool(first)), ctypes.c_void_p(_stream(stream))))


def dp_accumulate_all_range(plan: int, first: bool, begin: int, end: int, stream=None) -> None:
    _check(lib.dp_accumulate_all_range(ctypes.c_void_p(plan), int(bool(first)), begin, end,
                                       ctypes.c_void_p(_stream(stream))))


def dp_accumulate_reduce(plan: int, stream=None) -> None:
    _check(lib.dp_accumulate_reduce(ctypes.c_void_p(plan), ctypes.c_void_p(_stream(stream))))


def dp_accumulate_reduce_range(plan: int, begin: int, end: int, stream=None) -> None:
    _check(lib.dp_accumulate_reduce_range(ctypes.c_void_p(plan), begin, end, ctypes.c_void_p(_stream(stream))))


def dp_reduce_replicas(plan: int, src: int = DP_ROLE_ACC, stream=None) -> None:
    _check(lib.dp_reduce_replicas(ctypes.c_void_p(plan), src, ctypes.c_void_p(_stream(stream))))


def dp_reduce_replicas_range(plan: int, src: int, begin: int, end: int, stream=None) -> None:
    _check(lib.dp_reduce_replicas_range(ctypes.c_void_p(plan), src, begin, end, ctypes.c_void_p(_stream(stream))))


def dp_grad_stats(plan: int, scan: bool, max_norm: float = 0.0, stream=None) -> None:
    _check(lib.dp_grad_stats(ctypes.c_void_p(plan), int(bool(scan)), float(max_norm),
                             ctypes.c_void_p(_stream(stream))))


def dp_adam_step(plan: int, lr: float, eps: float, weight_decay: float, shard_begin: int, shard_end: int,
                 stream=None) -> None:
    hp = AdamHparams(lr, eps, weight_decay)
    _check(lib.dp_adam_step(ctypes.c_void_p(plan), ctypes.byref(hp), shard_begin, shard_end,
                            ctypes.c_void_p(_stream(stream))))


def dp_reduce_adam_step(plan: int, lr: float, eps: float, weight_decay: float, stream=None) -> None:
    hp = AdamHparams(lr, eps, weight_decay)
    _check(lib.dp_reduce_adam_step(ctypes.c_void_p(plan), ctypes.byref(hp), ctypes.c_void_p(_stream(stream))))


def dp_reduce_adam_step_noalloc(P: int, n: int, grad_dtype: str, param_dtype: str, grads: Sequence, accs,
                                master: Sequence, exp_avg: Sequence, exp_avg_sq: Sequence, param, state,
                                lr: float, eps: float, weight_decay: float, beta1: float, beta2: float,
                                scaler: str = "none", init_scale: float = 1.0, backoff: float = 0.5,
                                growth: float = 2.0, growth_interval: int = 2000, stream=None) -> None:
    """grads: n device buffers (tensors or addresses); accs: n buffers or
    None; master, exp_avg, exp_avg_sq: the two banks of each; state: device
    memory holding a dp_step_state."""
    def arr(xs):
        return (ctypes.c_void_p * max(1, len(xs)))(*[_addr(x) for x in xs])

    g = arr(list(grads))
    a = arr(list(accs)) if accs is not None else None
    banks = [arr(list(x)) for x in (master, exp_avg, exp_avg_sq)]
    cfg = StateCfg(beta1, beta2, SCALERS[scaler], growth_interval, init_scale, backoff, growth)
    hp = AdamHparams(lr, eps, weight_decay)
    pp = ctypes.POINTER(ctypes.c_void_p)
    _check(lib.dp_reduce_adam_step_noalloc(P, n, DTYPES[grad_dtype], DTYPES[param_dtype], g,
                                           a if a is not None else ctypes.cast(None, pp), *banks,
                                           ctypes.c_void_p(_addr(param)), ctypes.c_void_p(_addr(state)),
                                           ctypes.byref(cfg), ctypes.byref(hp), ctypes.c_void_p(_stream(stream))))


def dp_reduce_adam_range(plan: int, lr: float, eps: float, weight_decay: float, begin: int, end: int,
                         stream=None) -> None:
    hp = AdamHparams(lr, eps, weight_decay)
    _check(lib.dp_reduce_adam_range(ctypes.c_void_p(plan), ctypes.byref(hp), begin, end,
                                    ctypes.c_void_p(_stream(stream))))


def dp_reduce_adam_finish(plan: int, stream=None) -> None:
    _check(lib.dp_reduce_adam_finish(ctypes.c_void_p(plan), ctypes.c_void_p(_stream(stream))))


def dp_read_state(plan: int, stream=None) -> dict:
    st = StepState()
    _check(lib.dp_read_state(ctypes.c_void_p(plan), ctypes.byref(st), ctypes.c_void_p(_stream(stream))))
    return st.as_dict()


# ----------------------------------------------------------------------------
# checkpoints (dpckpt.h): host layer on numpy arrays, device layer on a plan
# ----------------------------------------------------------------------------
PARAM_NP = {"bf16": np.uint16, "f16": np.uint16}


def _layout(numel: Sequence[int], param_dtype: str):
    arr = (ctypes.c_int64 * max(len(numel), 1))(*[int(x) for x in numel])
    return Layout(len(numel), 1, arr, DP_BF16, DTYPES[param_dtype], 0, 0), arr


def _f32c(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a


def dp_ckpt_write_shard(directory: str, generation: int, numel: Sequence[int], param_dtype: str, begin: int,
                        end: int, master, exp_avg, exp_avg_sq, param) -> None:
    lay, keep = _layout(numel, param_dtype)
    arrs = [_f32c(master), _f32c(exp_avg), _f32c(exp_avg_sq), np.ascontiguousarray(param, dtype=np.uint16)]
    for a in arrs:
        if a.size != end - begin:
            raise ValueError(f"arrays must hold end - begin = {end - begin} elements, got {a.size}")
    ptrs = [a.ctypes.data_as(ctypes.c_void_p) for a in arrs]
    _check(lib.dp_ckpt_write_shard(os.fsencode(directory), generation, ctypes.byref(lay), begin, end, *ptrs))


def _state_struct(d: dict) -> "StepState":
    st = StepState()
    for k, _ in StepState._fields_:
        if k in d:
            setattr(st, k, d[k])
    return st


def dp_ckpt_commit(directory: str, generation: int, numel: Sequence[int], param_dtype: str, scalars: dict,
                   cfg: dict) -> None:
    lay, keep = _layout(numel, param_dtype)
    st = _state_struct(scalars)
    c = StateCfg(**cfg)
    _check(lib.dp_ckpt_commit(os.fsencode(directory), generation, ctypes.byref(lay), ctypes.byref(st),
                              ctypes.byref(c)))


def dp_ckpt_read(directory: str, numel: Sequence[int], param_dtype: str, begin: int, end: int,
                 arrays: bool = True) -> dict:
    """{'master', 'exp_avg', 'exp_avg_sq', 'param' (uint16 bits): [begin, end),
    'scalars': dict, 'cfg': dict, 'generation': int}"""
    lay, keep = _layout(numel, param_dtype)
    n = end - begin
    out = {}
    ptrs = [None] * 4
    if arrays:
        out = {"master": np.empty(n, np.float32), "exp_avg": np.empty(n, np.float32),
               "exp_avg_sq": np.empty(n, np.float32), "param": np.empty(n, np.uint16)}
        ptrs = [a.ctypes.data_as(ctypes.c_void_p) for a in out.values()]
    st, c, gen = StepState(), StateCfg(), ctypes.c_int64()
    _check(lib.dp_ckpt_read(os.fsencode(directory), ctypes.byref(lay), begin, end, *ptrs, ctypes.byref(st),
                            ctypes.byref(c), ctypes.byref(gen)))
    out["scalars"] = st.as_dict()
    out["cfg"] = {k: getattr(c, k) for k, _ in StateCfg._fields_}
    out["generation"] = int(gen.value)
    return out


def dp_checkpoint_save(plan: int, directory: str, generation: int, begin: int, end: int, stream=None) -> None:
    _check(lib.dp_checkpoint_save(ctypes.c_void_p(plan), os.fsencode(directory), generation, begin, end,
                                  ctypes.c_void_p(_stream(stream))))


def dp_checkpoint_commit(plan: int, directory: str, generation: int, stream=None) -> None:
    _check(lib.dp_checkpoint_commit(ctypes.c_void_p(plan), os.fsencode(directory), generation,
                                    ctypes.c_void_p(_stream(stream))))


def dp_checkpoint_load(plan: int, directory: str, begin: int, end: int, restore_scalars: bool,
                       stream=None) -> None:
    _check(lib.dp_checkpoint_load(ctypes.c_void_p(plan), os.fsencode(directory), begin, end,
                                  int(bool(restore_scalars)), ctypes.c_void_p(_stream(stream))))


# ----------------------------------------------------------------------------
# object wrapper
# ----------------------------------------------------------------------------
class Plan:
    """One plan over a ragged tensor list (see ``dpstep.h``)."""

    def __init__(self, numel: Sequence[int], n_replicas: int, grad_dtype: str = "bf16", param_dtype: str = "bf16",
                 chunk_elems: int = 0):
        self.numel = tuple(int(x) for x in numel)
        self.n = int(n_replicas)
        self.grad_dtype, self.param_dtype = grad_dtype, param_dtype
        self.handle = dp_plan_create(self.numel, self.n, grad_dtype, param_dtype, chunk_elems)
        self.P = int(sum(self.numel))

    def close(self) -> None:
        if self.handle:
            dp_plan_destroy(self.handle)
            self.handle = 0

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def info(self) -> dict:
        return dp_plan_info_get(self.handle)

    def chunks(self, begin: int = 0, end: Optional[int] = None) -> np.ndarray:
        return dp_plan_chunks(self.handle, begin, self.P if end is None else end)

    def bind(self, role: str, buf, replica: int = 0) -> None:
        dp_plan_bind_flat(self.handle, ROLES[role], replica, buf)

    def bind_tensors(self, role: str, bufs: Iterable, replica: int = 0) -> None:
        dp_plan_bind_tensors(self.handle, ROLES[role], replica, bufs, len(self.numel))

    def prepare_range(self, begin: int, end: int) -> None:
        dp_plan_prepare_range(self.handle, begin, end)

    def drop_ranges(self) -> None:
        dp_plan_drop_ranges(self.handle)

    def state_init(self, beta1: float = 0.9, beta2: float = 0.999, scaler: str = "none", init_scale: float = 1.0,
                   backoff: float = 0.5, growth: float = 2.0, growth_interval: int = 2000, stream=None) -> None:
        dp_state_init(self.handle, beta1, beta2, scaler, init_scale, backoff, growth, growth_interval, stream)

    def accumulate(self, replica: int, first: bool, emit_stats: bool = False, stream=None) -> None:
        dp_accumulate(self.handle, replica, first, emit_stats, stream)

    def accumulate_all(self, first: bool, stream=None) -> None:
        dp_accumulate_all(self.handle, first, stream)

    def accumulate_all_range(self, first: bool, begin: int, end: int, stream=None) -> None:
        dp_accumulate_all_range(self.handle, first, begin, end, stream)

    def accumulate_reduce(self, stream=None) -> None:
        dp_accumulate_reduce(self.handle, stream)

    def accumulate_reduce_range(self, begin: int, end: int, stream=None) -> None:
        dp_accumulate_reduce_range(self.handle, begin, end, stream)

    def reduce_replicas(self, src: str = "acc", stream=None) -> None:
        dp_reduce_replicas(self.handle, ROLES[src], stream)

    def reduce_replicas_range(self, src: str, begin: int, end: int, stream=None) -> None:
        dp_reduce_replicas_range(self.handle, ROLES[src], begin, end, stream)

    def grad_stats(self, scan: bool = False, max_norm: float = 0.0, stream=None) -> None:
        dp_grad_stats(self.handle, scan, max_norm, stream)

    def adam_step(self, lr: float, eps: float, weight_decay: float, begin: int = 0, end: Optional[int] = None,
                  stream=None) -> None:
        dp_adam_step(self.handle, lr, eps, weight_decay, begin, self.P if end is None else end, stream)

    def reduce_adam_step(self, lr: float, eps: float, weight_decay: float, stream=None) -> None:
        dp_reduce_adam_step(self.handle, lr, eps, weight_decay, stream)

    def reduce_adam_range(self, lr: float, eps: float, weight_decay: float, begin: int, end: int,
                          stream=None) -> None:
        dp_reduce_adam_range(self.handle, lr, eps, weight_decay, begin, end, stream)

    def reduce_adam_finish(self, stream=None) -> None:
        dp_reduce_adam_finish(self.handle, stream)

    def read_state(self, stream=None) -> dict:
        return dp_read_state(self.handle, stream)

    def checkpoint_save(self, directory: str, generation: int, begin: int = 0, end: Optional[int] = None,
                        stream=None) -> None:
        dp_checkpoint_save(self.handle, directory, generation, begin, self.P if end is None else end, stream)

    def checkpoint_commit(self, directory: str, generation: int, stream=None) -> None:
        dp_checkpoint_commit(self.handle, directory, generation, stream)

    def checkpoint_load(self, directory: str, begin: int = 0, end: Optional[int] = None,
                        restore_scalars: bool = True, stream=None) -> None:
        dp_checkpoint_load(self.handle, directory, begin, self.P if end is None else end, restore_scalars, stream)
