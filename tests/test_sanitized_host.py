"""The C-ABI layer's host code under AddressSanitizer (no GPU).

api.cpp and checkpoint.cpp are compiled for the host with the sanitizer and
linked with stub kernel launchers (tests/c/host_stubs.cpp) and the HIP
runtime.  Two C programs run against that build:
  * tests/c/abi_host.c: plan checks, chunk tables, bindings, order checks and
    the checkpoint host layer;
  * tests/c/ckpt_fuzz.c: seeded damage to a committed checkpoint (bytes
    flipped, ranges zeroed, files cut short), each read returning a status,
    and exact data whenever it returns DP_OK.
Any out-of-bounds access, use after free or leak fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gradient_reduce_adam_amd", "csrc")
SAN = "-fsanitize=address"


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    gxx, gcc = shutil.which("g++"), shutil.which("gcc")
    if not (gxx and gcc and os.path.isdir("/opt/rocm/include")):
        pytest.skip("needs g++, gcc and the ROCm headers")
    out = tmp_path_factory.mktemp("asan")
    inc = ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
    cxx = [gxx, "-std=c++17", SAN, "-fno-omit-frame-pointer", "-g", "-O1"] + inc
    objs = []
    for src in (os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "checkpoint.cpp"),
                os.path.join(ROOT, "tests", "c", "host_stubs.cpp")):
        obj = str(out / (os.path.basename(src) + ".o"))
        r = subprocess.run(cxx + ["-c", src, "-o", obj], capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, r.stderr[-4000:]
        objs.append(obj)
    exes = {}
    for name in ("abi_host", "ckpt_fuzz"):
        obj = str(out / (name + ".o"))
        r = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", SAN, "-g"] + inc[:3] +
                           ["-c", os.path.join(ROOT, "tests", "c", name + ".c"), "-o", obj],
                           capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, r.stderr[-4000:]
        exe = str(out / name)
        r = subprocess.run([gxx, SAN, obj] + objs + ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
                                                     "-o", exe], capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, r.stderr[-4000:]
        exes[name] = exe
    return out, exes


def _run(args):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=99")
    return subprocess.run(args, capture_output=True, text=True, timeout=600, env=env)


def test_host_calls_clean_under_asan(sanitized):
    out, exes = sanitized
    d = out / "abi_ckpt"
    d.mkdir()
    r = _run([exes["abi_host"], str(d)])
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout[-2000:] + r.stderr[-4000:]


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_damaged_checkpoints_clean_under_asan(sanitized, seed):
    out, exes = sanitized
    d = out / f"fuzz{seed}"
    d.mkdir()
    r = _run([exes["ckpt_fuzz"], str(d), "1500", str(seed)])
    assert r.returncode == 0 and r.stdout.startswith("ok "), r.stdout[-2000:] + r.stderr[-4000:]
    reads, detected = map(int, r.stdout.split()[1:3])
    assert reads == 1500 and 0 < detected < reads
