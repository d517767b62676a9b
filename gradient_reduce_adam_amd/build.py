"""Builds the gfx950 shared library ``libdpstep.so`` in place with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libdpstep.so")

HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             # packed binary32 arithmetic stays off: the streaming kernels are
             # bound by HBM, not by the vector ALUs
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-result"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed: " + " ".join(cmd) + "\n" + r.stdout)
    return r.stdout


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "csrc")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", src]
    objs = []
    for name in ("kernels.hip", "api.cpp", "checkpoint.cpp", "noalloc.hip"):
        obj = os.path.join(src, name + ".o")
        out = _run(["hipcc", *HIP_FLAGS, *inc, "-c", os.path.join(src, name), "-o", obj])
        if verbose and out:
            sys.stdout.write(out)
        objs.append(obj)
    _run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"])
    os.replace(LIB + ".tmp", LIB)
    for o in objs:
        os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
