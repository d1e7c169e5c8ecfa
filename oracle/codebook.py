"""Lloyd-Max scalar quantizers for the standard normal, frozen as fp16 centroids.

TQ-MSE (review page, §1 Key Terms; abstract) rotates a vector and quantizes coordinates
with a distortion-optimal scalar quantizer whose error falls as 4^-b.  No page fixes the
table.  Reading used here: for b = 1..8 bits the table is the Lloyd-Max quantizer of
N(0, 1) (centroid = conditional mean of its cell, thresholds = midpoints), with each
centroid rounded to the nearest fp16 value and each threshold the exact midpoint of two
adjacent fp16 centroids (exact in fp32).

The fixed point is found by Newton's method on c = G(c), G the Lloyd map, using the
symmetric positive half; the Jacobian of G is tridiagonal.
"""
from __future__ import annotations

import functools
import math

import numpy as np
from scipy.special import erfc, ndtri

B_MAX = 8
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


def _pdf(x):
    return np.exp(-0.5 * x * x) * _INV_SQRT_2PI


def _upper_tail(x):
    """Q(x) = P(X >= x) for X ~ N(0,1)."""
    return 0.5 * erfc(x / math.sqrt(2.0))


def _cells(c_pos: np.ndarray):
    """Thresholds of the positive half: 0, midpoints, +inf."""
    h = len(c_pos)
    t = np.empty(h + 1)
    t[0] = 0.0
    t[1:h] = 0.5 * (c_pos[:-1] + c_pos[1:])
    t[h] = np.inf
    return t


def _lloyd_map(c_pos: np.ndarray):
    """Conditional means of the positive cells and their derivatives w.r.t. the cell ends."""
    t = _cells(c_pos)
    a, b = t[:-1], t[1:]
    last = np.isinf(b)
    bf = np.where(last, 0.0, b)
    fa, fb = _pdf(a), np.where(last, 0.0, _pdf(bf))
    # phi(a) - phi(b) without cancellation: phi(a) * (1 - exp(-(b-a)(b+a)/2))
    num = np.where(last, fa, -fa * np.expm1(-0.5 * (bf - a) * (bf + a)))
    mass = np.where(last, _upper_tail(a), _upper_tail(a) - _upper_tail(bf))
    mu = num / mass
    dmu_da = fa / mass * (mu - a)
    dmu_db = np.where(last, 0.0, fb / mass * (bf - mu))
    return mu, dmu_da, dmu_db


def lloyd_max_fp64(b: int) -> np.ndarray:
    """All 2^b Lloyd-Max centroids of N(0,1), ascending, float64."""
    if not 1 <= b <= B_MAX:
        raise ValueError("b must be in 1..8")
    n, h = 2 ** b, 2 ** (b - 1)
    c = ndtri((np.arange(h) + 0.5) / n + 0.5)  # start: centres of equiprobable cells
    for _ in range(100):
        mu, da, db = _lloyd_map(c)
        # Newton step on F(c) = G(c) - c: (I - J_G) x = G(c) - c, J_G tridiagonal.
        sub = np.zeros(h); dia = np.ones(h); sup = np.zeros(h)
        sub[1:] = -0.5 * da[1:]
        dia[1:] -= 0.5 * da[1:]
        dia[:-1] -= 0.5 * db[:-1]
        sup[:-1] = -0.5 * db[:-1]
        rhs = mu - c
        cp = np.zeros(h); dp = np.zeros(h)
        cp[0], dp[0] = sup[0] / dia[0], rhs[0] / dia[0]
        for k in range(1, h):
            m = dia[k] - sub[k] * cp[k - 1]
            cp[k] = sup[k] / m
            dp[k] = (rhs[k] - sub[k] * dp[k - 1]) / m
        x = np.zeros(h)
        x[-1] = dp[-1]
        for k in range(h - 2, -1, -1):
            x[k] = dp[k] - cp[k] * x[k + 1]
        c = c + x
        if np.max(np.abs(x)) < 1e-13:
            break
    return np.concatenate([-c[::-1], c])


@functools.lru_cache(maxsize=None)
def codebook(b: int):
    """(centroids fp16 [2^b] ascending, thresholds fp32 [2^b - 1]) of the frozen b-bit table."""
    c16 = lloyd_max_fp64(b).astype(np.float16)
    c64 = c16.astype(np.float64)
    mid = 0.5 * (c64[:-1] + c64[1:])
    thr = mid.astype(np.float32)
    assert np.array_equal(thr.astype(np.float64), mid), "midpoint not exact in fp32"
    c16.setflags(write=False)
    thr.setflags(write=False)
    return c16, thr


def codebook_mse(b: int) -> float:
    """Exact mean squared error of the frozen b-bit table for X ~ N(0,1) (closed form per cell:
    E[(X-c)^2; a<=X<b] = P + a*phi(a) - b*phi(b) - 2c(phi(a)-phi(b)) + c^2 P)."""
    c16, thr = codebook(b)
    c = c16.astype(np.float64)
    edges = np.concatenate([[-np.inf], thr.astype(np.float64), [np.inf]])
    total = 0.0
    for m in range(len(c)):
        a, e = edges[m], edges[m + 1]
        pa = 0.0 if np.isinf(a) else _pdf(a)
        pe = 0.0 if np.isinf(e) else _pdf(e)
        mass = _upper_tail(a) - _upper_tail(e)
        apa = 0.0 if np.isinf(a) else a * pa
        epe = 0.0 if np.isinf(e) else e * pe
        total += mass + apa - epe - 2 * c[m] * (pa - pe) + c[m] ** 2 * mass
    return float(total)
