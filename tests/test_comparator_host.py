"""The tolerance comparison the GPU parity tests use (gpu_common), on the
CPU: values within the stated tolerance pass, values outside it fail, a
non-finite value matches only a non-finite value of the same kind, the
binary32 ulp bound catches what the absolute floor lets through, and under
clipping m may differ by what the norm's summation order allows, no more."""
import numpy as np
import pytest

from gpu_common import MAX_ULP_CLIPPED, assert_state_close, oracle_run, ulps32
from test_gpu_random_configs import _draw

LOOSE = 1 << 30  # ulp bound that never binds: the stated tolerance alone


def _state(w):
    w = np.asarray(w, dtype=np.float32)
    return {"w": w, "m": w.copy(), "v": w.copy(), "p": np.zeros(w.size, np.uint16)}


def _up(x, k):
    """x moved up by k binary32 ulp."""
    x = np.float32(x)
    for _ in range(k):
        x = np.nextafter(x, np.float32(np.inf))
    return x


@pytest.mark.parametrize("got,ref", [
    ([1.0], [1.0]),
    ([np.nextafter(np.float32(1), np.float32(2))], [1.0]),  # 1 ulp: 1.2e-7 relative
    ([np.inf, -np.inf], [np.inf, -np.inf]),
    ([np.nan], [np.nan]),
    ([0.0], [5e-10]),  # the absolute floor
])
def test_matches(got, ref):
    assert_state_close(_state(got), _state(ref), LOOSE, where="match")


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
        assert_state_close(_state(got), _state(ref), LOOSE, where="mismatch")


def test_ulp_bound_zero_demands_equal_bits():
    ref = [0.02, -3e-14, 7e-13]
    assert_state_close(_state(ref), _state(ref), 0, where="equal")
    for i in range(3):
        got = np.array(ref, np.float32)
        got[i] = _up(got[i], 1)
        with pytest.raises(AssertionError, match="ulp"):
            assert_state_close(_state(got), _state(ref), 0, where="one ulp")


def test_ulp_bound_catches_values_below_the_absolute_floor():
    """A second moment of 3e-14 (the size v has after one step of the
    gpt2_small workload) passes the stated tolerance when it is lost
    entirely or doubled, since both errors sit below the 1e-9 floor; the ulp
    bound fails both."""
    ref = [3e-14]
    for got in ([0.0], [6e-14]):
        assert_state_close(_state(got), _state(ref), LOOSE, where="floor only")
        with pytest.raises(AssertionError, match="ulp"):
            assert_state_close(_state(got), _state(ref), MAX_ULP_CLIPPED, where="with ulp bound")


def test_ulp_bound_with_clipping():
    """64 ulp is 7.6e-6 relative, looser than the stated 2e-6 for values above
    the absolute floor; the bound binds for the small moments below it."""
    ref = np.array([1e-12, -2e-11, 3e-14], np.float32)
    near = np.array([_up(x, MAX_ULP_CLIPPED) for x in ref], np.float32)
    far = np.array([_up(x, MAX_ULP_CLIPPED + 1) for x in ref], np.float32)
    rep = assert_state_close(_state(near), _state(ref), MAX_ULP_CLIPPED, where="at the bound")
    assert rep["w_max_ulp"] == MAX_ULP_CLIPPED
    with pytest.raises(AssertionError, match="ulp"):
        assert_state_close(_state(far), _state(ref), MAX_ULP_CLIPPED, where="past the bound")


def test_ulp_distance_crosses_zero():
    """+0 and -0 are 0 ulp apart; the smallest subnormals of either sign 2."""
    tiny = np.float32(1e-45)
    assert_state_close(_state([0.0]), _state([-0.0]), 0, where="signed zero")
    rep = assert_state_close(_state([tiny]), _state([-tiny]), 2, where="across zero")
    assert rep["m_max_ulp"] == 2


def test_nonfinite_pairs_are_not_ulp_counted():
    """NaNs of different payloads are the same kind; their bit distance is
    not an ulp distance."""
    a = np.array([np.nan], np.float32)
    b = np.array([0x7FC00001], np.uint32).view(np.float32)
    assert_state_close(_state(a), _state(b), 0, where="nan payloads")


def test_m_slack_exempts_only_m_and_only_within_it():
    ref = _state([1e-13, 0.01, 0.02])
    ref["m_slack"] = np.array([1e-18, 1e-18, 1e-18])
    got = _state([1e-13, 0.01, 0.02])
    got["m"][0] = _up(np.float32(1e-13), 200)  # 200 ulp, 1.3e-18 absolute: beyond the slack
    with pytest.raises(AssertionError, match="ulp"):
        assert_state_close(got, ref, MAX_ULP_CLIPPED, where="beyond slack")
    got["m"][0] = _up(np.float32(1e-13), 100)  # 100 ulp, 6.3e-19 absolute: within it
    rep = assert_state_close(got, ref, MAX_ULP_CLIPPED, where="within slack")
    assert rep["m_max_ulp"] == 100 and rep["m_within_norm_order_slack"] == 1
    got["w"][0] = got["m"][0]  # the same difference in w is not exempt
    with pytest.raises(AssertionError, match="w: 1 elements more than"):
        assert_state_close(got, ref, MAX_ULP_CLIPPED, where="w")


def test_m_slack_covers_the_norms_summation_order():
    """The oracle against itself with the norm's binary64 sum taken in
    another order (chunks of 777 elements instead of 2^20), on a clipped
    configuration of the random sweep (5 partials, clip 1.0, a NaN that skips
    step 1) where m nearly cancels at one element: there m moves by more than
    64 ulp, everywhere it stays within the slack, and w and v stay within the
    ulp bound."""
    w, *_ = _draw(1851)
    a = oracle_run(w, w.steps)
    b = oracle_run(w, w.steps, chunk=777)
    A, B = a.state[(0, w.P)], b.state[(0, w.P)]
    assert any(x["norm"] != y["norm"] for x, y in zip(a.scalars, b.scalars))  # the orders differ
    u = ulps32(A["m"], B["m"])
    assert u.max() > MAX_ULP_CLIPPED
    d = np.abs(A["m"].astype(np.float64) - B["m"].astype(np.float64))
    assert np.all(d <= A["m_slack"]) and np.all(d <= B["m_slack"])
    for k in ("w", "v"):
        assert ulps32(A[k], B[k]).max() <= MAX_ULP_CLIPPED, k
    assert_state_close(B, A, MAX_ULP_CLIPPED, where="two norm orders")
