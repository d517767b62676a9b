"""The tolerance comparison the GPU parity tests use (gpu_common), on the
CPU: values within the stated tolerance pass, values outside it fail, and a
non-finite value matches only a non-finite value of the same kind."""
import numpy as np
import pytest

from gpu_common import assert_state_close


def _state(w):
    w = np.asarray(w, dtype=np.float32)
    return {"w": w, "m": w.copy(), "v": w.copy(), "p": np.zeros(w.size, np.uint16)}


@pytest.mark.parametrize("got,ref", [
    ([1.0], [1.0]),
    ([np.nextafter(np.float32(1), np.float32(2))], [1.0]),  # 1 ulp: 1.2e-7 relative
    ([np.inf, -np.inf], [np.inf, -np.inf]),
    ([np.nan], [np.nan]),
    ([0.0], [5e-10]),  # the absolute floor
])
def test_matches(got, ref):
    assert_state_close(_state(got), _state(ref), where="match")


@pytest.mark.parametrize("got,ref", [
    ([1.001], [1.0]),
    ([np.inf], [-np.inf]),
    ([np.nan], [1.0]),
    ([1.0], [np.nan]),
    ([np.inf], [3.0e38]),
    ([3.0e38], [np.inf]),
    ([np.nan], [np.inf]),
])
def test_mismatches(got, ref):
    with pytest.raises(AssertionError):
        assert_state_close(_state(got), _state(ref), where="mismatch")
