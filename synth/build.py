"""Builds the two compiled twins of the input generator in place:
``libsynth_host.so`` (gcc, OpenMP) and ``libsynth_gpu.so`` (hipcc, gfx950)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed: " + " ".join(cmd) + "\n" + r.stdout)


def build(gpu: bool = True) -> None:
    src = os.path.join(HERE, "csrc")
    _run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          os.path.join(src, "synth_host.c"), "-o", os.path.join(HERE, "libsynth_host.so")])
    if gpu:
        _run(["hipcc", *HIP_FLAGS, os.path.join(src, "synth_gpu.hip"), "-o", os.path.join(HERE, "libsynth_gpu.so")])


if __name__ == "__main__":
    build()
