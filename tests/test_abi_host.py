"""The C-ABI library on the host: it loads, exports every symbol its header
declares, and its host-side logic (layout checks, chunk tables, byte model,
argument and ordering errors) behaves as documented.  No compute call is made
here: everything below fails validation before touching a GPU, or is host
work by contract."""
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]

dp = pytest.importorskip("gradient_reduce_adam_amd")


def _declared():
    text = "".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(dp_\w+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) == 32, names
    assert sorted(dp.EXPORTS) == names
    for n in names:
        assert hasattr(dp.lib, n), n


def test_abi_version_and_status_strings():
    assert dp.dp_abi_version() == 3
    assert dp.dp_status_string(dp.DP_ERR_RANGE) == "range out of bounds"
    assert dp.dp_status_string(0) == "ok"
    # every status has a string in the library and a name in the binding
    for st in range(dp.DP_ERR_CORRUPT + 1):
        assert dp.dp_status_string(st) != "unknown status"
        assert dp.DpError(st, "x").args[0].startswith("DP_")
    assert dp.dp_status_string(dp.DP_ERR_CORRUPT + 1) == "unknown status"


@pytest.mark.parametrize("kw", [dict(n_replicas=0), dict(n_replicas=17), dict(grad_dtype="f32"),
                                dict(param_dtype="f32"), dict(chunk_elems=100), dict(chunk_elems=1 << 27),
                                dict(chunk_elems=768)])
def test_bad_layouts_rejected(kw):
    args = dict(numel=[10, 20], n_replicas=2, grad_dtype="bf16", param_dtype="bf16", chunk_elems=0)
    args.update(kw)
    with pytest.raises(dp.DpError) as e:
        dp.dp_plan_create(**args)
    assert e.value.status == dp.DP_ERR_BAD_LAYOUT


def test_negative_numel_rejected():
    with pytest.raises(dp.DpError) as e:
        dp.dp_plan_create([5, -1], 1, "bf16", "bf16")
    assert e.value.status == dp.DP_ERR_BAD_LAYOUT and "numel[1]" in e.value.message


def _brute_chunks(numel, chunk, begin, end):
    out = []
    pos = 0
    for t, n in enumerate(numel):
        for off in range(0, n, chunk):
            lo, hi = pos + off, pos + min(n, off + chunk)
            a, b = max(lo, begin), min(hi, end)
            if a < b:
                out.append((a, a - pos, t, b - a))
        pos += n
    return out


@pytest.mark.parametrize("numel,chunk", [((1000, 0, 3, 70000, 256, 65536, 65537), 256),
                                         ((1 << 20,), 65536), ((5, 5, 5), 256), ((), 256)])
def test_chunk_table_matches_brute_force(numel, chunk):
    with dp.Plan(numel, 1, "bf16", "bf16", chunk) as p:
        P = sum(numel)
        rng = np.random.default_rng(3)
        ranges = [(0, P), (0, 0)] + [tuple(sorted(rng.integers(0, P + 1, 2))) for _ in range(20)] if P else [(0, 0)]
        for b, e in ranges:
            got = p.chunks(int(b), int(e))
            ref = _brute_chunks(numel, chunk, int(b), int(e))
            assert [tuple(int(x) for x in r) for r in got] == ref


try:
    from hypothesis import given, settings, strategies as st
except ImportError:  # pragma: no cover
    given = None

if given is not None:
    @settings(max_examples=300, deadline=None)
    @given(numel=st.lists(st.integers(0, 5000), max_size=12), log2c=st.integers(8, 13),
           cut=st.tuples(st.floats(0, 1), st.floats(0, 1)))
    def test_chunk_table_property(numel, log2c, cut):
        """Random ragged layouts (empty tensors included), every power-of-two
        chunk size from 256 to 8192, random ranges: the library's table equals
        the brute-force one, and its chunks tile the range."""
        chunk = 1 << log2c
        P = sum(numel)
        b, e = sorted(int(c * P) for c in cut)
        with dp.Plan(numel, 1, "bf16", "bf16", chunk) as p:
            got = [tuple(int(x) for x in r) for r in p.chunks(b, e)]
        assert got == _brute_chunks(numel, chunk, b, e)
        assert sum(r[3] for r in got) == e - b
        assert all(0 < r[3] <= chunk for r in got)


def test_chunk_table_of_a_2pow32_tensor_uses_64bit_indices():
    with dp.Plan((1 << 32, 7), 4, "f16", "f16", 65536) as p:
        c = p.chunks()
        assert len(c) == (1 << 32) // 65536 + 1
        assert int(c[-2]["flat"]) == (1 << 32) - 65536 and int(c[-1]["flat"]) == 1 << 32
        assert int(c[-1]["offset"]) == 0 and int(c[-1]["tensor"]) == 1 and int(c[-1]["len"]) == 7
        mid = p.chunks((1 << 31) + 5, (1 << 31) + 70000)
        assert int(mid[0]["offset"]) == (1 << 31) + 5 and int(mid[0]["len"]) == 65531
    with dp.Plan((1 << 32,), 1, "bf16", "bf16") as p:
        assert p.info()["chunk_elems"] == dp.DP_DEFAULT_CHUNK == 16384
        assert p.info()["num_chunks"] == (1 << 32) // 16384


def test_plan_info_byte_model():
    numel = (50257 * 768, 768, 3)
    with dp.Plan(numel, 8, "bf16", "bf16") as p:
        info = p.info()
        P = sum(numel)
        assert info["params"] == P and info["num_tensors"] == 3 and info["n_replicas"] == 8
        assert info["state_bytes"] == 16 * P
        assert info["bytes_accumulate_first"] == 6 * P and info["bytes_accumulate"] == 10 * P
        assert info["bytes_reduce_acc"] == (4 * 8 + 4) * P and info["bytes_reduce_partials"] == (2 * 8 + 4) * P
        assert info["bytes_adam"] == 30 * P and info["bytes_stats_scan"] == 4 * P
        assert info["bytes_accumulate_reduce"] == ((2 + 4) * 8 + 4) * P
        assert info["bytes_reduce_adam"] == ((2 + 4) * 8 + 26) * P
        assert info["bytes_reduce_adam_partials"] == (2 * 8 + 26) * P
        assert info["num_chunks"] == len(p.chunks())


def test_bind_and_call_errors_before_any_launch():
    with dp.Plan((1000, 24), 2, "bf16", "bf16") as p:
        h = p.handle
        with pytest.raises(dp.DpError) as e:
            dp.dp_plan_bind_flat(h, 9, 0, 0x1000)
        assert e.value.status == dp.DP_ERR_INVALID_ARG
        with pytest.raises(dp.DpError) as e:
            dp.dp_plan_bind_flat(h, dp.DP_ROLE_ACC, 2, 0x1000)
        assert e.value.status == dp.DP_ERR_INVALID_ARG
        with pytest.raises(dp.DpError) as e:
            dp.dp_plan_bind_flat(h, dp.DP_ROLE_MASTER, 2, 0x1000)  # two banks only
        assert e.value.status == dp.DP_ERR_INVALID_ARG
        with pytest.raises(dp.DpError) as e:
            dp.dp_plan_bind_flat(h, dp.DP_ROLE_PARAM, 1, 0x1000)  # one PARAM buffer
        assert e.value.status == dp.DP_ERR_INVALID_ARG
        with pytest.raises(dp.DpError) as e:
            dp.dp_accumulate(h, 0, True, stream=0)
        assert e.value.status == dp.DP_ERR_UNBOUND
        dp.dp_plan_bind_flat(h, dp.DP_ROLE_GRAD, 0, 0x1000)
        dp.dp_plan_bind_flat(h, dp.DP_ROLE_ACC, 0, 0x2000)
        with pytest.raises(dp.DpError) as e:
            dp.dp_accumulate(h, 0, False, stream=0)  # no first micro-step yet
        assert e.value.status == dp.DP_ERR_STATE
        with pytest.raises(dp.DpError) as e:
            dp.dp_accumulate(h, 0, True, emit_stats=True, stream=0)  # n = 2
        assert e.value.status == dp.DP_ERR_INVALID_ARG
        with pytest.raises(dp.DpError) as e:
            dp.dp_accumulate(h, 2, True, stream=0)
        assert e.value.status == dp.DP_ERR_INVALID_ARG
        with pytest.raises(dp.DpError) as e:
            dp.dp_grad_stats(h, False, 1.0, stream=0)
        assert e.value.status == dp.DP_ERR_STATE
        with pytest.raises(dp.DpError) as e:
            dp.dp_accumulate_all(h, True, stream=0)  # GRAD of replica 1 unbound
        assert e.value.status == dp.DP_ERR_UNBOUND
        with pytest.raises(dp.DpError) as e:
            dp.dp_accumulate_reduce(h, stream=0)  # before dp_state_init
        assert e.value.status == dp.DP_ERR_STATE
        with pytest.raises(dp.DpError) as e:
            dp.dp_reduce_replicas(h, dp.DP_ROLE_ACC, stream=0)
        assert e.value.status == dp.DP_ERR_STATE
        with pytest.raises(dp.DpError) as e:
            dp.dp_reduce_replicas(h, dp.DP_ROLE_MASTER, stream=0)
        assert e.value.status == dp.DP_ERR_INVALID_ARG
        for b, e_ in ((-1, 10), (5, 4), (0, 1025)):
            with pytest.raises(dp.DpError) as e:
                dp.dp_adam_step(h, 1e-3, 1e-8, 0.0, b, e_, stream=0)
            assert e.value.status == dp.DP_ERR_RANGE
        with pytest.raises(dp.DpError) as e:
            dp.dp_adam_step(h, 1e-3, 0.0, 0.0, 0, 10, stream=0)
        assert e.value.status == dp.DP_ERR_INVALID_ARG
        with pytest.raises(dp.DpError) as e:
            dp.dp_adam_step(h, 1e-3, 1e-8, 0.0, 0, 10, stream=0)  # no statistics yet
        assert e.value.status == dp.DP_ERR_STATE
        with pytest.raises(dp.DpError) as e:
            dp.dp_reduce_adam_step(h, 1e-3, 1e-8, 0.0, stream=0)  # before dp_state_init
        assert e.value.status == dp.DP_ERR_STATE
        with pytest.raises(dp.DpError) as e:
            dp.dp_reduce_adam_step(h, 1e-3, -1.0, 0.0, stream=0)
        assert e.value.status == dp.DP_ERR_INVALID_ARG
        with pytest.raises(dp.DpError) as e:
            dp.dp_read_state(h, stream=0)
        assert e.value.status == dp.DP_ERR_STATE
        with pytest.raises(dp.DpError) as e:
            dp.dp_plan_chunks(h, 0, 2000)
        assert e.value.status == dp.DP_ERR_RANGE
        assert "not inside" in dp.dp_last_error()


def test_ranged_call_errors_before_any_launch():
    with dp.Plan((1000, 24), 2, "bf16", "bf16") as p:
        h = p.handle
        with pytest.raises(dp.DpError) as e:
            dp.dp_accumulate_all_range(h, True, 0, 256, stream=0)  # nothing bound
        assert e.value.status == dp.DP_ERR_UNBOUND
        for r in range(2):
            dp.dp_plan_bind_flat(h, dp.DP_ROLE_GRAD, r, 0x1000 * (r + 1))
            dp.dp_plan_bind_flat(h, dp.DP_ROLE_ACC, r, 0x10000 * (r + 1))
        with pytest.raises(dp.DpError) as e:
            dp.dp_accumulate_all_range(h, False, 0, 256, stream=0)  # no first micro-step yet
        assert e.value.status == dp.DP_ERR_STATE
        for b, e_ in ((-1, 256), (512, 256), (0, 1025)):
            with pytest.raises(dp.DpError) as e:
                dp.dp_accumulate_all_range(h, True, b, e_, stream=0)
            assert e.value.status == dp.DP_ERR_RANGE
        with pytest.raises(dp.DpError) as e:
            dp.dp_reduce_replicas_range(h, dp.DP_ROLE_MASTER, 0, 256, stream=0)
        assert e.value.status == dp.DP_ERR_INVALID_ARG
        with pytest.raises(dp.DpError) as e:
            dp.dp_reduce_replicas_range(h, dp.DP_ROLE_ACC, 0, 256, stream=0)  # before dp_state_init
        assert e.value.status == dp.DP_ERR_STATE


def test_bind_tensors_checks_the_pointer_count():
    with dp.Plan((1000, 24, 7), 1, "bf16", "bf16") as p:
        for bad in ([0x1000, 0x2000], [0x1000] * 4):
            with pytest.raises(ValueError):
                p.bind_tensors("master", bad)
            with pytest.raises(ValueError):  # the low-level call asks the plan
                dp.dp_plan_bind_tensors(p.handle, dp.DP_ROLE_MASTER, 0, bad)


def test_destroy_null_is_ok():
    dp.dp_plan_destroy(0)


def test_headers_are_c_and_host_calls_work_from_c(tmp_path):
    """Both headers compile as C99 with warnings as errors, and a C program
    linked against the library makes the host-only calls: plan checks, the
    chunk table, bindings, and a checkpoint written in two shards and read
    back across them (tests/c/abi_host.c)."""
    import os
    import shutil
    import subprocess

    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    libdir = os.path.join(root, "gradient_reduce_adam_amd")
    exe = tmp_path / "abi_host"
    cc = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                         "-I" + os.path.join(root, "include"), "-I/opt/rocm/include",
                         os.path.join(root, "tests", "c", "abi_host.c"), "-o", str(exe), "-L" + libdir, "-ldpstep",
                         "-Wl,-rpath," + libdir, "-Wl,-rpath,/opt/rocm/lib"], capture_output=True, text=True)
    assert cc.returncode == 0, cc.stderr[-4000:]
    (tmp_path / "ckpt").mkdir()
    r = subprocess.run([str(exe), str(tmp_path / "ckpt")], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr


@pytest.mark.parametrize("P", [-1, dp.DP_STATIC_MAX_PARAMS + 1, 1 << 40])
def test_noalloc_rejects_sizes_outside_its_scratch(P):
    """The allocation-free single pass checks the size against its static
    scratch before it touches a GPU (the addresses are never used)."""
    fake = 1 << 20
    with pytest.raises(dp.DpError) as e:
        dp.dp_reduce_adam_step_noalloc(P, 1, "bf16", "bf16", [fake], None, [fake, fake], [fake, fake],
                                       [fake, fake], fake, fake, 1e-3, 1e-8, 0.01, 0.9, 0.999, stream=0)
    assert e.value.status == dp.DP_ERR_INVALID_ARG
    if P > 0:
        assert "DP_STATIC_MAX_PARAMS" in e.value.message


def test_noalloc_scratch_size_matches_its_layout():
    """The header's scratch size is the sum of its parts for 2^30 elements:
    binary64 sums and 32-bit counts per 256-element piece, binary64 sums and
    64-bit counts per 4096 pieces, and one 24-byte chunk entry per 16384
    elements."""
    pieces = dp.DP_STATIC_MAX_PARAMS // 256
    assert dp.DP_STATIC_SCRATCH_BYTES == pieces * 12 + (pieces // 4096) * 16 + \
        (dp.DP_STATIC_MAX_PARAMS // dp.DP_DEFAULT_CHUNK) * 24
