"""Pins for the oracle's per-row quantities: the log-normaliser of softmax(z/T) and the argmax.

p = softmax(z/T) is the temperature step of SDCP's sampling profile ("Speculative Decoding
Coordination Protocol (SDCP)", section "Session Contract"); the argmax with the smallest id on ties
is its temperature-zero rule.  The oracle's LSE is checked against a closed form, against a
50-digit mpmath evaluation and against scipy's logsumexp; the argmax against planted ties.
"""
import math

import mpmath
import numpy as np
import pytest
from scipy.special import logsumexp

from oracle import oracle
from workloads import bf16_bits, bf16_to_f32


@pytest.mark.parametrize("V", [1, 8, 1000, 128256])
@pytest.mark.parametrize("T", [1.0, 0.8, 0.25, 3.0])
@pytest.mark.parametrize("c", [0.0, -2.5, 7.0])
def test_lse_constant_row_closed_form(V, T, c):
    row = np.full(V, c, dtype=np.float32)
    assert oracle.row_lse(row, T) == pytest.approx(c / T + math.log(V), rel=0, abs=1e-12 * max(1.0, abs(c / T)))
    rowb = bf16_bits(row)
    assert oracle.row_lse(rowb, T) == pytest.approx(float(bf16_to_f32(rowb)[0]) / T + math.log(V), abs=1e-11)


def test_lse_matches_mpmath_50_digits():
    mpmath.mp.dps = 50
    rng = np.random.default_rng(11)
    for trial in range(40):
        V = int(rng.integers(1, 40))
        T = float(rng.choice([1.0, 0.8, 0.3, 2.0]))
        row = (rng.standard_normal(V) * rng.choice([0.5, 3.0, 20.0])).astype(np.float32)
        exact = mpmath.log(mpmath.fsum(mpmath.exp(mpmath.mpf(float(z)) / T) for z in row))
        assert abs(oracle.row_lse(row, T) - float(exact)) < 1e-13 * max(1.0, abs(float(exact)))


@pytest.mark.parametrize("V", [32000, 128256, 151936])
def test_lse_matches_scipy_logsumexp(V):
    rng = np.random.default_rng(V)
    row = (rng.standard_normal(V) * 3.0).astype(np.float32)
    rowb = bf16_bits(row)
    for T in (1.0, 0.8):
        ref = logsumexp(bf16_to_f32(rowb).astype(np.float64) / T)
        assert oracle.row_lse(rowb, T) == pytest.approx(ref, rel=1e-14, abs=1e-12)


def test_lse_handles_minus_infinity():
    row = np.array([-np.inf, 0.0, -np.inf, 1.0], dtype=np.float32)
    assert oracle.row_lse(row, 1.0) == pytest.approx(math.log(1.0 + math.e), abs=1e-15)
    assert oracle.row_lse(np.full(5, -np.inf, dtype=np.float32), 1.0) == -np.inf


def test_argmax_smallest_index_on_ties():
    rng = np.random.default_rng(5)
    for _ in range(200):
        V = int(rng.integers(1, 3000))
        row = bf16_bits(rng.standard_normal(V).astype(np.float32))
        vals = bf16_to_f32(row)
        m = vals.max()
        k = int(rng.integers(1, 6))
        planted = np.sort(rng.choice(V, size=min(k, V), replace=False))
        vals = vals.copy()
        vals[planted] = m + 1.0
        rowb = bf16_bits(vals)
        assert oracle.row_argmax(rowb) == int(planted[0])
        assert oracle.row_argmax(bf16_to_f32(rowb)) == int(np.argmax(bf16_to_f32(rowb)))


def test_argmax_ties_are_frequent_in_bf16_rows():
    # at the greedy workload's scale (N(0, 4^2), V = 151936) bf16 rounding makes exact ties common;
    # the oracle must agree with numpy's first-occurrence argmax on every one of them
    rng = np.random.default_rng(3)
    ties = 0
    for _ in range(64):
        rowb = bf16_bits((rng.standard_normal(151936) * 4.0).astype(np.float32))
        vals = bf16_to_f32(rowb)
        ties += int((vals == vals.max()).sum() > 1)
        assert oracle.row_argmax(rowb) == int(np.argmax(vals))
    assert ties > 0
