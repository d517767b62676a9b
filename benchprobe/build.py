"""Builds ``libbenchprobe.so`` (hipcc, gfx950) in place."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build() -> str:
    out = os.path.join(HERE, "libbenchprobe.so")
    cmd = ["hipcc", *HIP_FLAGS, os.path.join(HERE, "csrc", "probes.hip"), "-o", out + ".tmp"]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed: " + " ".join(cmd) + "\n" + r.stdout)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build())
