import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: a workload at full size (tens of seconds of oracle time)")


def _ensure_built():
    """Builds only what is missing (the round's build step compiles
    everything; tests load what is built)."""
    oracle_lib = os.path.join(ROOT, "oracle", "liboracle.so")
    synth_host = os.path.join(ROOT, "synth", "libsynth_host.so")
    if not os.path.exists(oracle_lib):
        from oracle import build as ob
        ob.build()
    if not os.path.exists(synth_host):
        from synth import build as sb
        sb.build(gpu=False)


_ensure_built()


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


def pytest_collection_modifyitems(config, items):
    if gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
