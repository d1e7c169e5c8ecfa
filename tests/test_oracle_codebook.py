"""Pins for oracle.codebook (Lloyd-Max N(0,1) tables frozen to fp16)."""
import math
import os

import numpy as np
import pytest
from scipy import integrate

from oracle import codebook as cb

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "lloyd_max_gaussian.txt")


def _golden():
    rows = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        b, cents, thr, mse = [f.strip() for f in line.split("|")]
        rows[int(b)] = ([float(x) for x in cents.split()], [float(x) for x in thr.split()], float(mse))
    return rows


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_textbook_values(b):
    cents, thr, mse = _golden()[b]
    c64 = cb.lloyd_max_fp64(b)
    pos = c64[len(c64) // 2:]
    # 4 significant digits as printed
    for got, want in zip(pos, cents):
        assert abs(got - want) <= 0.6 * 10 ** (math.floor(math.log10(want)) - 3), (got, want)
    t64 = 0.5 * (pos[:-1] + pos[1:])
    for got, want in zip(t64, thr):
        assert abs(got - want) <= 0.6 * 10 ** (math.floor(math.log10(want)) - 3), (got, want)
    # frozen (fp16-rounded) table: MSE within 0.1% of the unrounded optimum
    assert abs(cb.codebook_mse(b) - mse) / mse < 1e-3


def test_b1_closed_form():
    c16, thr = cb.codebook(1)
    assert c16[1] == np.float16(math.sqrt(2 / math.pi)) and c16[0] == -c16[1]
    assert thr[0] == 0.0
    assert abs(cb.codebook_mse(1) - (1 - 2 / math.pi)) < 1e-6


@pytest.mark.parametrize("b", range(1, 9))
def test_fixed_point_by_quadrature(b):
    """Each fp64 centroid is the conditional mean of its cell (quadrature, not the erfc formula)."""
    c = cb.lloyd_max_fp64(b)
    edges = np.concatenate([[-np.inf], 0.5 * (c[:-1] + c[1:]), [np.inf]])
    pdf = lambda x: math.exp(-0.5 * x * x) / math.sqrt(2 * math.pi)
    for m in range(len(c) // 2, len(c)):  # positive half (symmetry checked below)
        lo, hi = edges[m], edges[m + 1]
        mass = integrate.quad(pdf, lo, hi, epsabs=0, epsrel=1e-13)[0]
        first = integrate.quad(lambda x: x * pdf(x), lo, hi, epsabs=0, epsrel=1e-13)[0]
        assert abs(first / mass - c[m]) < 1e-9 * max(1.0, abs(c[m]))


@pytest.mark.parametrize("b", range(1, 9))
def test_symmetry_rounding_and_thresholds(b):
    c64 = cb.lloyd_max_fp64(b)
    c16, thr = cb.codebook(b)
    assert len(c16) == 2 ** b and len(thr) == 2 ** b - 1
    assert np.array_equal(c16, -c16[::-1])
    assert np.all(np.diff(c16.astype(np.float64)) > 0)
    # nearest fp16
    for x, h in zip(c64, c16):
        nxt = np.nextafter(h, np.float16(np.inf)); prv = np.nextafter(h, np.float16(-np.inf))
        assert abs(float(h) - x) <= abs(float(nxt) - x) and abs(float(h) - x) <= abs(float(prv) - x)
    mids = 0.5 * (c16[:-1].astype(np.float64) + c16[1:].astype(np.float64))
    assert np.array_equal(thr.astype(np.float64), mids)
    assert thr[(len(thr) - 1) // 2] == 0.0


@pytest.mark.parametrize("b", [2, 5, 8])
def test_mse_closed_form_vs_quadrature(b):
    c16, thr = cb.codebook(b)
    c = c16.astype(np.float64)
    edges = np.concatenate([[-np.inf], thr.astype(np.float64), [np.inf]])
    pdf = lambda x: math.exp(-0.5 * x * x) / math.sqrt(2 * math.pi)
    tot = sum(integrate.quad(lambda x, cm=c[m]: (x - cm) ** 2 * pdf(x), edges[m], edges[m + 1],
                             epsabs=1e-15, epsrel=1e-12)[0] for m in range(len(c)))
    assert abs(tot - cb.codebook_mse(b)) < 1e-10


def test_rate_4_pow_minus_b():
    """Distortion falls by ~4x per bit and D(b)*4^b rises toward the Panter-Dite constant."""
    D = [cb.codebook_mse(b) for b in range(1, 9)]
    scaled = [D[b - 1] * 4 ** b for b in range(1, 9)]
    assert all(np.diff(scaled) > 0)
    assert abs(scaled[-1] - math.pi * math.sqrt(3) / 2) / (math.pi * math.sqrt(3) / 2) < 0.01
    for b in range(2, 9):
        assert 3.0 < D[b - 2] / D[b - 1] < 4.0


@pytest.mark.parametrize("b", [1, 3, 6])
def test_monte_carlo_mse(b):
    c16, thr = cb.codebook(b)
    x = np.random.default_rng(b).standard_normal(1_000_000)
    code = np.searchsorted(thr.astype(np.float64), x, side="right")
    err = (x - c16.astype(np.float64)[code]) ** 2
    D = cb.codebook_mse(b)
    assert abs(err.mean() - D) < 5 * err.std() / math.sqrt(len(x))
