"""Pins for the oracle's specified fp32 exponential (Cody-Waite reduction + Taylor).

The routing weights must be reproducible bit for bit, so the exponential is specified
rather than taken from a library; these tests pin it to the mathematics: every fp32 in
the routing range is within 2 ulp of the correctly rounded exp, exact at 0, zero below
the cut-off, and monotone.
"""
import math

import numpy as np
import pytest

import oracle


def test_exact_points():
    assert oracle.exp32([0.0])[0] == np.float32(1.0)
    assert oracle.exp32([-0.0])[0] == np.float32(1.0)
    # below the cut-off the result is +0 (weight contribution below 2^-125 of the max)
    y = oracle.exp32([-87.0001, -100.0, -1e30])
    assert np.all(y == 0.0) and not np.any(np.signbit(y))
    y87 = oracle.exp32([-87.0])[0]
    assert y87 > 0 and y87 >= np.finfo(np.float32).tiny  # never subnormal


@pytest.mark.parametrize("x", [-1.0, -0.5, -math.log(2.0), -10.0, -20.5, -86.9])
def test_against_fp64(x):
    got = float(oracle.exp32([x])[0])
    ref = math.exp(float(np.float32(x)))
    assert abs(got - ref) <= 2 * np.spacing(np.float32(ref))


def test_exhaustive_routing_range():
    # every fp32 in [-87, 0]: about 1.1e9 values, checked in C with OpenMP
    err, worst = oracle.exp_max_ulp(-87.0, 0.0)
    assert err <= 2.0, (err, worst)


def test_monotone_dense_sample():
    bits = np.arange(0x80000000, 0xC2AE0000, 4099, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)  # -0 .. -87, decreasing x
    y = oracle.exp32(x)
    assert np.all(np.diff(y) <= 0)
