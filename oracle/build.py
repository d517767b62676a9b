"""Builds the CPU oracle (``liboracle.so``) in place with gcc.

Test infrastructure: building the checker is not using it."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def build() -> None:
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           os.path.join(HERE, "oracle.c"), "-o", os.path.join(HERE, "liboracle.so"), "-lm"]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + r.stdout)


if __name__ == "__main__":
    build()
