"""Seeded synthetic inputs for the data-parallel update step.

This package is the only code shared by the oracle side and the GPU side of
the tests and the benchmark.  It generates inputs (initial master weights and
per-replica, per-micro-step gradients) and describes the workloads; it holds
none of the update step's arithmetic.

Generator definition (implemented three times, bit-identically: pure Python
below for tiny counts, C in ``csrc/synth_host.c``, HIP in
``csrc/synth_gpu.hip``):

* ``mix64`` is the SplitMix64 output function (Steele, Lea & Flood 2014).
* ``key(seed, role, step, replica, micro)`` hashes the stream coordinates.
* position ``i`` of a stream hashes ``key + (i + 1) * GOLDEN``; the four 16-bit
  fields of that hash sum to an Irwin-Hall(4) integer ``z`` in
  ``[-131070, 131070]`` whose standard deviation is ``65536 / sqrt(3)``.
* the binary32 value is ``RNE(float(z) * c)`` with ``c = f32(sigma * sqrt(3) /
  65536 * multiplier * loss_scale)``, then rounded to nearest-even into the
  output format.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB_PATH = os.path.join(_HERE, "libsynth_host.so")
GPU_LIB_PATH = os.path.join(_HERE, "libsynth_gpu.so")

MASK64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15

ROLE_MASTER = 1
ROLE_GRAD = 2
ROLE_SELECT = 3

DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2}


# ----------------------------------------------------------------------------
# pure-Python definition (tiny counts; pins the compiled twins)
# ----------------------------------------------------------------------------
def mix64(z: int) -> int:
    z &= MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def stream_key(seed: int, role: int, step: int, replica: int, micro: int) -> int:
    fields = ((role & 0xFF) << 56) | ((step & 0xFFFFFF) << 32) | ((replica & 0xFFFF) << 16) | (micro & 0xFFFF)
    return mix64(mix64((seed + GOLDEN) & MASK64) ^ fields)


def hash_at(key: int, i: int) -> int:
    return mix64((key + (i + 1) * GOLDEN) & MASK64)


def irwin_hall_int(key: int, i: int) -> int:
    h = hash_at(key, i)
    return (h & 0xFFFF) + ((h >> 16) & 0xFFFF) + ((h >> 32) & 0xFFFF) + ((h >> 48) & 0xFFFF) - 131070


def scale_constant(sigma: float, multiplier: float = 1.0, loss_scale: float = 1.0) -> np.float32:
    """The binary32 constant ``c`` that maps the Irwin-Hall integer to a draw
    of standard deviation ``sigma * multiplier`` times ``loss_scale``."""
    return np.float32(sigma * math.sqrt(3.0) / 65536.0 * multiplier * loss_scale)


def py_normal(key: int, start: int, count: int, c: np.float32, dtype: str) -> np.ndarray:
    """Pure-Python/NumPy reference of the generator for small ``count``.

    Conversion to binary16 uses NumPy's ``astype`` (round to nearest even);
    conversion to bfloat16 rounds the binary32 bits to nearest even by integer
    arithmetic."""
    z = np.array([irwin_hall_int(key, start + j) for j in range(count)], dtype=np.int64)
    x = z.astype(np.float32) * np.float32(c)  # one binary32 multiply, RNE
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    u = x.view(np.uint32).astype(np.uint64)
    out = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


# ----------------------------------------------------------------------------
# compiled twins
# ----------------------------------------------------------------------------
_host = None
_gpu = None


def _host_lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB_PATH):
            raise ImportError(f"{HOST_LIB_PATH} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(HOST_LIB_PATH)
        lib.synth_stream_key.restype = ctypes.c_uint64
        lib.synth_stream_key.argtypes = [ctypes.c_uint64] + [ctypes.c_uint32] * 4
        lib.synth_hash_at.restype = ctypes.c_uint64
        lib.synth_hash_at.argtypes = [ctypes.c_uint64, ctypes.c_int64]
        lib.synth_normal_host.restype = None
        lib.synth_normal_host.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
                                          ctypes.c_int, ctypes.c_void_p, ctypes.c_int]
        _host = lib
    return _host


def _gpu_lib():
    global _gpu
    if _gpu is None:
        if not os.path.exists(GPU_LIB_PATH):
            raise ImportError(f"{GPU_LIB_PATH} is not built; run __graft_entry__.build()")
        import torch  # noqa: F401  (load torch's HIP runtime first: one runtime per process)
        lib = ctypes.CDLL(GPU_LIB_PATH)
        lib.synth_normal_device.restype = ctypes.c_int
        lib.synth_normal_device.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
                                            ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        lib.synth_poke_u16.restype = ctypes.c_int
        lib.synth_poke_u16.argtypes = [ctypes.c_void_p, ctypes.c_uint32, ctypes.c_void_p]
        lib.synth_normal_device_multi.restype = ctypes.c_int
        lib.synth_normal_device_multi.argtypes = [ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(ctypes.c_void_p),
                                                  ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
                                                  ctypes.c_int, ctypes.c_void_p]
        _gpu = lib
    return _gpu


def host_stream_key(seed: int, role: int, step: int, replica: int, micro: int) -> int:
    return int(_host_lib().synth_stream_key(seed, role, step, replica, micro))


def host_hash_at(key: int, i: int) -> int:
    return int(_host_lib().synth_hash_at(key, i))


def host_normal(key: int, start: int, count: int, c: np.float32, dtype: str, out: Optional[np.ndarray] = None,
                threads: int = 1) -> np.ndarray:
    """C host twin: ``count`` values from stream position ``start``.

    Returns float32 for ``dtype == 'f32'`` and the raw uint16 bit patterns for
    ``'f16'`` and ``'bf16'``."""
    npdt = np.float32 if dtype == "f32" else np.uint16
    if out is None:
        out = np.empty(count, dtype=npdt)
    assert out.dtype == npdt and out.size >= count and out.flags.c_contiguous
    if count:
        _host_lib().synth_normal_host(key, start, count, float(c), DTYPE_CODES[dtype],
                                      out.ctypes.data, int(threads))
    return out


def device_normal(key: int, start: int, count: int, c: np.float32, dtype: str, out_ptr: int, stream: int) -> None:
    """HIP twin: writes ``count`` values from stream position ``start`` to the
    device buffer at ``out_ptr``, asynchronously on ``stream``."""
    rc = _gpu_lib().synth_normal_device(key, start, count, float(c), DTYPE_CODES[dtype],
                                        ctypes.c_void_p(out_ptr), ctypes.c_void_p(stream))
    if rc != 0:
        raise RuntimeError(f"synth_normal_device failed with code {rc}")


# ----------------------------------------------------------------------------
# workload-level helpers
# ----------------------------------------------------------------------------
def master_key(w) -> int:
    return stream_key(w.seed, ROLE_MASTER, 0, 0, 0)


def grad_key(w, step: int, replica: int, micro: int) -> int:
    return stream_key(w.seed, ROLE_GRAD, step, replica, micro)


def master_host(w, lo: int, hi: int, threads: int = 1) -> np.ndarray:
    """Initial binary32 master weights on the flat range [lo, hi)."""
    return host_normal(master_key(w), lo, hi - lo, scale_constant(w.master_sigma), "f32", threads=threads)


def _injected(w, step, replica, micro, lo, hi):
    for (s, r, k, idx, val) in w.injections:
        if s == step and r == replica and k == micro and lo <= idx < hi:
            yield idx, val


def _lp_bits(val: float, dtype: str) -> int:
    x = np.array([val], dtype=np.float32)
    if dtype == "f16":
        return int(x.astype(np.float16).view(np.uint16)[0])
    u = int(x.view(np.uint32)[0])
    return u >> 16 if (u & 0x7F800000) != 0x7F800000 or (u & 0x7FFFFF) == 0 else (u >> 16) | 0x40


def grad_host(w, step: int, replica: int, micro: int, lo: int, hi: int, loss_scale: float,
              threads: int = 1, out: Optional[np.ndarray] = None) -> np.ndarray:
    """Stored gradient bits (uint16) of one replica and micro-step on [lo, hi)."""
    from .workloads import grad_segments
    if out is None:
        out = np.empty(hi - lo, dtype=np.uint16)
    key = grad_key(w, step, replica, micro)
    for start, count, c in grad_segments(w, lo, hi, loss_scale):
        host_normal(key, start, count, c, w.grad_dtype, out=out[start - lo:start - lo + count], threads=threads)
    for idx, val in _injected(w, step, replica, micro, lo, hi):
        out[idx - lo] = _lp_bits(val, w.grad_dtype)
    return out


def grad_device(w, step: int, replica: int, micro: int, out_ptr: int, loss_scale: float, stream: int,
                lo: int = 0, hi: Optional[int] = None) -> None:
    """Same values as ``grad_host`` written to the device buffer ``out_ptr``
    (element 0 of the buffer is flat index ``lo``)."""
    from .workloads import grad_segments
    hi = w.P if hi is None else hi
    key = grad_key(w, step, replica, micro)
    for start, count, c in grad_segments(w, lo, hi, loss_scale):
        device_normal(key, start, count, c, w.grad_dtype, out_ptr + 2 * (start - lo), stream)
    for idx, val in _injected(w, step, replica, micro, lo, hi):
        _poke_u16(out_ptr + 2 * (idx - lo), _lp_bits(val, w.grad_dtype), stream)


def master_device(w, out_ptr: int, stream: int, lo: int = 0, hi: Optional[int] = None) -> None:
    hi = w.P if hi is None else hi
    device_normal(master_key(w), lo, hi - lo, scale_constant(w.master_sigma), "f32", out_ptr, stream)


def grads_device_replicas(w, step: int, micro: int, slots, loss_scale: float, stream: int, lo: int = 0,
                          hi: Optional[int] = None) -> None:
    """``grad_device`` for every replica at once (one launch per piece of
    [lo, hi)), into slots[r] + 2 * lo for replica r: the same values."""
    from .workloads import grad_segments
    hi = w.P if hi is None else hi
    n = w.n
    keys = (ctypes.c_uint64 * n)(*[grad_key(w, step, r, micro) for r in range(n)])
    for start, count, c in grad_segments(w, lo, hi, loss_scale):
        outs = (ctypes.c_void_p * n)(*[slots[r] + 2 * start for r in range(n)])
        rc = _gpu_lib().synth_normal_device_multi(keys, outs, n, start, count, float(c), DTYPE_CODES[w.grad_dtype],
                                                  ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"synth_normal_device_multi failed with code {rc}")
    for r in range(n):
        for idx, val in _injected(w, step, r, micro, lo, hi):
            _poke_u16(slots[r] + 2 * idx, _lp_bits(val, w.grad_dtype), stream)


def _poke_u16(ptr: int, bits: int, stream: int) -> None:
    rc = _gpu_lib().synth_poke_u16(ctypes.c_void_p(ptr), bits, ctypes.c_void_p(stream))
    if rc != 0:
        raise RuntimeError(f"synth_poke_u16 failed with code {rc}")


from .workloads import Workload  # noqa: E402,F401  (re-export)
