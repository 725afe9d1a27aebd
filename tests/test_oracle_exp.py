"""Pins of the oracle's fp32 exp and sigmoid against fp64 exp (numpy/libm).

The router's scoring is this build's reading (sigmoid; the pages name only
an FP32 gate bias).  exp is written from Cody-Waite range reduction and a
Taylor polynomial; these tests bound its error against the correctly rounded
value over the whole range it is used on, and check exact special values.
"""
import numpy as np

import oracle


def _ulp_err(got32: np.ndarray, ref64: np.ndarray) -> np.ndarray:
    ref32 = ref64.astype(np.float32)
    ulp = np.spacing(np.abs(ref32)).astype(np.float64)
    return np.abs(got32.astype(np.float64) - ref64) / ulp


def _sweep(lo_bits: int, hi_bits: int, stride: int) -> np.ndarray:
    return np.arange(lo_bits, hi_bits, stride, dtype=np.uint32).view(np.float32)


def test_exp_error_over_range_strided():
    # positive side (0, 88.5) and negative side (-86, 0): every 251st fp32 value
    pos = _sweep(0x00000001, 0x42B10000, 251)
    neg = -_sweep(0x00000001, 0x42AC0000, 251)
    for y in (pos, neg):
        got = oracle.exp(y)
        err = _ulp_err(got, np.exp(y.astype(np.float64)))
        assert err.max() <= 2.0, err.max()
        assert np.mean(err <= 1.0) > 0.999


def test_exp_error_exhaustive_on_one_binade():
    y = _sweep(0x3F000000, 0x3F800000, 1)  # every fp32 in [0.5, 1)
    err = _ulp_err(oracle.exp(y), np.exp(y.astype(np.float64)))
    assert err.max() <= 2.0
    y = -y
    err = _ulp_err(oracle.exp(y), np.exp(y.astype(np.float64)))
    assert err.max() <= 2.0


def test_exp_special_values_and_saturation():
    assert oracle.exp(np.float32(0.0))[()] == 1.0
    assert oracle.exp(np.float32(-0.0))[()] == 1.0
    assert np.isinf(oracle.exp(np.float32(88.5))[()])
    assert np.isinf(oracle.exp(np.float32(1000.0))[()])
    assert oracle.exp(np.float32(-86.0))[()] == 0.0
    assert oracle.exp(np.float32(-1e30))[()] == 0.0
    # just inside the thresholds the result is a finite normal number
    below = np.nextafter(np.float32(88.5), np.float32(0))
    above = np.nextafter(np.float32(-86.0), np.float32(0))
    assert np.isfinite(oracle.exp(below)[()])
    assert oracle.exp(above)[()] >= np.finfo(np.float32).tiny


def test_exp_monotone():
    y = np.sort(np.concatenate([-_sweep(1, 0x42AC0000, 997), _sweep(1, 0x42B10000, 997)]))
    e = oracle.exp(y)
    assert np.all(np.diff(e.astype(np.float64)) >= 0)


def test_sigmoid_values():
    assert oracle.sigmoid(np.float32(0.0))[()] == 0.5
    assert oracle.sigmoid(np.float32(86.0))[()] == 1.0
    assert oracle.sigmoid(np.float32(-88.5))[()] == 0.0
    y = np.linspace(-40, 40, 200001, dtype=np.float32)
    got = oracle.sigmoid(y)
    ref = 1.0 / (1.0 + np.exp(-y.astype(np.float64)))
    assert _ulp_err(got, ref).max() <= 3.0
    assert np.all(np.diff(got.astype(np.float64)) >= 0)
    # symmetry s(-l) = 1 - s(l) up to rounding
    assert np.max(np.abs(oracle.sigmoid(-y).astype(np.float64) + got - 1.0)) < 2e-7
