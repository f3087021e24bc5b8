"""The scoring kernels' erf (no GPU): Abramowitz and Stegun, Handbook of
Mathematical Functions, formula 7.1.26, with the constants exactly as typed in
the device source, against math.erf.  The handbook bounds the formula's
absolute error by 1.5e-7; the layer's reading of the pages allows a named
published approximation of erf within 1e-6."""
import math
import os
import re

import numpy as np

SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "learnable_kv_cache_amd", "csrc",
                   "score_core.h")


def _constants():
    text = open(SRC).read()
    names = ["kErfP", "kErfA1", "kErfA2", "kErfA3", "kErfA4", "kErfA5"]
    vals = {}
    for n in names:
        m = re.search(r"constexpr float %s = (-?[0-9.]+)f;" % n, text)
        assert m, n
        vals[n] = float(m.group(1))
    return vals


def _erf_as(x, c, dtype):
    """The device formula, evaluated in dtype (float32 mirrors the kernel's arithmetic
    up to the reciprocal's and the exponential's last-bit errors)."""
    x = np.asarray(x, dtype)
    ax = np.abs(x)
    one = dtype(1.0)
    t = one / (dtype(c["kErfP"]) * ax + one)
    poly = t * (dtype(c["kErfA1"]) + t * (dtype(c["kErfA2"]) + t * (dtype(c["kErfA3"]) + t * (
        dtype(c["kErfA4"]) + t * dtype(c["kErfA5"])))))
    return np.copysign(one - poly * np.exp(-ax * ax), x)


def test_constants_are_the_handbooks():
    c = _constants()
    assert c == {"kErfP": 0.3275911, "kErfA1": 0.254829592, "kErfA2": -0.284496736,
                 "kErfA3": 1.421413741, "kErfA4": -1.453152027, "kErfA5": 1.061405429}


def test_error_bound_in_exact_arithmetic():
    c = _constants()
    x = np.linspace(-8.0, 8.0, 200001)
    ref = np.array([math.erf(v) for v in x])
    err = np.abs(_erf_as(x, c, np.float64) - ref)
    assert err.max() <= 1.5e-7 + 1e-12, err.max()


def test_error_in_float32_and_gelu():
    c = _constants()
    x = np.linspace(-8.0, 8.0, 200001)
    ref = np.array([math.erf(v) for v in x])
    err = np.abs(_erf_as(x, c, np.float32).astype(np.float64) - ref)
    assert err.max() <= 6e-7, err.max()                 # + float32 rounding of the steps
    # GELU(h) = h/2 (1 + erf(h/sqrt 2)): the erf error enters scaled by |h|/2
    h = np.linspace(-6.0, 6.0, 20001)
    g_dev = 0.5 * h * (1.0 + _erf_as(h / math.sqrt(2.0), c, np.float32).astype(np.float64))
    g_ref = np.array([0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))) for v in h])
    assert np.abs(g_dev - g_ref).max() <= 2e-6


def test_odd_and_limits():
    c = _constants()
    x = np.linspace(0.0, 10.0, 1001)
    np.testing.assert_array_equal(_erf_as(-x, c, np.float64), -_erf_as(x, c, np.float64))
    assert _erf_as(np.array([0.0]), c, np.float64)[0] == 0.0 or abs(
        _erf_as(np.array([0.0]), c, np.float64)[0]) <= 1.5e-7
    assert abs(_erf_as(np.array([10.0]), c, np.float64)[0] - 1.0) <= 1e-12
