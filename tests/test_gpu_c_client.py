"""The C ABI from C on the GPU: tests/c/step_gpu.c, a C99 program linked
against libdpstep.so and the HIP runtime only (no torch, its own buffers and
stream), runs two whole steps of a ragged workload with clipping, the update
split into two shard calls, and again with every micro-step and the
reduction in two buckets.  Its state and scalars must match the oracle's run
on the same seeded inputs, under the stated tolerances, and the two runs
must agree bit for bit."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import gradient_reduce_adam_amd as dp
import synth
from synth import workloads

from gpu_common import assert_scalars_match, assert_state_close, log, oracle_run, ulp_bound

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RAGGED = (3000, 17, 4096, 5, 70001, 256, 1, 65536, 131075)


def _build(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    libdir = os.path.join(ROOT, "gradient_reduce_adam_amd")
    exe = tmp_path / "step_gpu"
    cc = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                         "-I" + os.path.join(ROOT, "include"), "-I/opt/rocm/include",
                         os.path.join(ROOT, "tests", "c", "step_gpu.c"), "-o", str(exe), "-L" + libdir, "-ldpstep",
                         "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath," + libdir, "-Wl,-rpath,/opt/rocm/lib"],
                        capture_output=True, text=True, timeout=120)
    assert cc.returncode == 0, cc.stderr[-4000:]
    return exe


def test_c_program_runs_whole_steps_through_the_abi(tmp_path):
    results = {mode: _run_c_program(tmp_path, mode) for mode in ("whole", "buckets")}
    for k in ("w", "m", "v", "p"):
        assert np.array_equal(results["whole"][k].view(np.uint8), results["buckets"][k].view(np.uint8)), k


def _run_c_program(tmp_path, mode):
    w = workloads.gpt2_small().with_(numel=RAGGED, n=3, a=2, max_norm=0.05, scaled_tensors=(4,), param_dtype="f16",
                                     steps=2)
    P, steps = w.P, w.steps
    cut = int(w.offsets[4]) + 1000  # inside tensor 4
    exe = _build(tmp_path)
    d = tmp_path / f"io_{mode}"
    d.mkdir()
    dtypes = {"f16": dp.DP_F16, "bf16": dp.DP_BF16}
    with open(d / "config.txt", "w") as f:
        f.write(f"{P} {w.T} {w.n} {w.a} {steps} {dtypes[w.grad_dtype]} {dtypes[w.param_dtype]} {w.max_norm!r} "
                f"{w.lr!r} {w.eps!r} {w.weight_decay!r} {w.beta1!r} {w.beta2!r}\n")
        f.write(" ".join(str(x) for x in w.numel) + f"\n{cut}\n")
    synth.master_host(w, 0, P).astype(np.float32).tofile(d / "master.bin")
    grads = np.empty((steps, w.a, w.n, P), np.uint16)
    for s in range(steps):
        for k in range(w.a):
            for r in range(w.n):
                grads[s, k, r] = synth.grad_host(w, s + 1, r, k + 1, 0, P, 1.0)
    grads.tofile(d / "grads.bin")
    log(f"C client ({mode}): P={P} n={w.n} a={w.a} steps={steps} shards [0, {cut}) [{cut}, {P})")
    r = subprocess.run([str(exe), str(d)] + (["buckets"] if mode == "buckets" else []), capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr

    raw = np.fromfile(d / "state.bin", dtype=np.uint8)
    assert raw.size == 14 * P
    f32 = raw[:12 * P].view(np.float32)
    got = {"w": f32[:P], "m": f32[P:2 * P], "v": f32[2 * P:], "p": raw[12 * P:].view(np.uint16)}
    fields = open(d / "scalars.txt").read().split()
    scal = {"t": int(fields[0]), "iter": int(fields[1]), "growth_tracker": int(fields[2]),
            "found_inf": int(fields[3]), "beta1_pow": float.fromhex(fields[4]),
            "beta2_pow": float.fromhex(fields[5]), "scale": float.fromhex(fields[6]),
            "norm": float.fromhex(fields[7]), "clip": float.fromhex(fields[8])}

    ref = oracle_run(w, steps)
    assert scal["clip"] < 1.0 and scal["t"] == steps  # clipping was active on applied steps
    assert_scalars_match(scal, ref.scalars[-1], where="C client")
    rep = assert_state_close(got, ref.state[(0, P)], ulp_bound(w), where=f"C client ({mode})")
    log(f"  C client ({mode}) max ulp: {rep}")
    return got
