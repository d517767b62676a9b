"""Benchmark-only GPU kernels, none of them part of the method: bandwidth
references for ``bench.py`` (a copy, a read, and the stream mixes of the
library's streaming kernels) and a matrix-core load that stands in for the
compute of a backward pass (``bench.py --overlap``).  The library, the
oracle and the input generators never import this package."""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbenchprobe.so")

_lib = None


def lib():
    global _lib
    if _lib is None:
        try:
            import torch  # noqa: F401  (one HIP runtime: torch's)
        except ImportError:
            pass
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, PP = ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)
        L.probe_stream.argtypes = [ctypes.c_int, vp, vp, ctypes.c_int64, vp]
        L.probe_mix.argtypes = [ctypes.c_int] * 5 + [PP, PP, PP, PP, ctypes.c_int64, vp, vp]
        L.probe_busy.argtypes = [ctypes.c_double, vp]
        for f in (L.probe_stream, L.probe_mix, L.probe_busy):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{what} failed with code {rc}")


def stream(kind: str, src_ptr: int, dst_ptr: int, nbytes: int, stream: int) -> None:
    """One pass of the copy ("copy") or read ("read") reference."""
    _check(lib().probe_stream({"copy": 0, "read": 1}[kind], ctypes.c_void_p(src_ptr), ctypes.c_void_p(dst_ptr),
                              int(nbytes), ctypes.c_void_p(stream)), "probe_stream")


def mix(r16: Sequence[int], r32: Sequence[int], w32: Sequence[int], w16: Sequence[int], n: int, stream: int,
        rmw: bool = False, stagger: int = 0) -> None:
    """One pass of a stream mix over n elements: reads the 16-bit streams r16
    and binary32 streams r32, writes binary32 streams w32 and 16-bit streams
    w16 (device addresses); with rmw, r32[0] is w32[0], read and written in
    place.  stagger: device address of ceil(n / 16384) zero int64 entries that
    each wave loads before its first access, or 0."""
    def arr(xs):
        return (ctypes.c_void_p * max(1, len(xs)))(*[int(x) for x in xs])

    _check(lib().probe_mix(len(r16), len(r32), len(w32), len(w16), int(bool(rmw)), arr(r16), arr(r32), arr(w32),
                           arr(w16), int(n), ctypes.c_void_p(stagger), ctypes.c_void_p(stream)), "probe_mix")


def busy(flops: float, stream: int) -> None:
    """About `flops` bf16 matrix-core operations on `stream`, touching no memory."""
    _check(lib().probe_busy(float(flops), ctypes.c_void_p(stream)), "probe_busy")


# Backward-pass compute per parameter and token: about twice the forward's
# 2 flops per parameter and token.
BACKWARD_FLOPS_PER_PARAM_TOKEN = 4.0


def backward_bucket(w, step: int, micro: int, lo: int, hi: int, slots, loss_scale: float, stream: int,
                    tokens: int) -> None:
    """A synthetic backward pass over the parameters [lo, hi): the matrix-core
    compute of one replica's backward for those parameters at `tokens` tokens
    per micro-batch, then every replica's gradients of [lo, hi) written into
    its slot (slots[r]: device address of replica r's gradient buffer, which
    holds the whole flat space) by the seeded generator."""
    import synth

    busy(BACKWARD_FLOPS_PER_PARAM_TOKEN * (hi - lo) * tokens, stream)
    synth.grads_device_replicas(w, step, micro, slots, loss_scale, stream, lo, hi)
