"""CPU tests of the comparison rule itself (no GPU, no oracle)."""
import numpy as np

from tests import _compare


def _f16(v):
    return np.array(v, dtype=np.float64).astype(np.float16)


def test_within_and_outside_tolerance():
    x = np.array([0.0, 1000.0, -3.0])
    r = _f16(x)
    assert _compare.check(_f16([0.0099, 1001.9, -3.015]), r, x)[0] == 0
    assert _compare.check(_f16([0.02, 1000.0, -3.0]), r, x)[0] == 1
    assert _compare.check(_f16([0.0, 1004.0, -3.0]), r, x)[0] == 1


def test_nan_always_fails():
    x = np.array([1.0])
    assert _compare.check(_f16([np.nan]), _f16(x), x)[0] == 1


def test_overflow_rules():
    x = np.array([65400.0, 65510.0, 70000.0, -70000.0, 70000.0, 65530.0])
    r = _f16(x)                                       # 65408, 65504, inf, -inf, inf, inf
    y = _f16([65408.0, np.inf, np.inf, -np.inf, 65504.0, 65504.0])
    n, _, detail = _compare.check(y, r, x)
    assert n == 1, detail                             # 70000 must be inf, not 65504
    y2 = _f16([65408.0, -np.inf, np.inf, -np.inf, np.inf, 65504.0])
    assert _compare.check(y2, r, x)[0] == 1           # wrong sign in the band
