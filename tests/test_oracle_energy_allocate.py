"""Pins for oracle.energy (block energy, sigma) and oracle.allocate (greedy widths)."""
import itertools
import math

import numpy as np
import pytest

import synth
from oracle import allocate, energy


# ---------------------------------------------------------------- energy
def test_known_answer_block_pairing():
    """All key energy placed in coordinates (6, 7) lands in block 3 only; (2i, 2i+1) pairing."""
    T, d = 10, 128
    k = np.zeros((T, d)); q = np.zeros((2, T, d))
    k[:, 6] = np.arange(T); k[:, 7] = 1.0
    q[0, :, 64] = 2.0; q[1, :, 65] = 4.0
    ek, eq = energy.block_energy(k, q)
    want = np.mean(np.arange(T) ** 2 + 1.0)
    assert ek[3] == pytest.approx(want) and np.count_nonzero(ek) == 1
    assert eq[32] == pytest.approx((4.0 + 16.0) / 2) and np.count_nonzero(eq) == 1


def test_rope_invariance():
    """Rotating every block by any angle (RoPE at arbitrary positions) leaves energies unchanged."""
    rng = np.random.default_rng(0)
    k = rng.standard_normal((64, 128)) * np.repeat(rng.uniform(0.1, 5, 64), 2)
    q = rng.standard_normal((4, 64, 128))
    ek0, eq0 = energy.block_energy(k, q)
    pos = rng.integers(0, 10 ** 6, 64)
    ek1, eq1 = energy.block_energy(synth.rope(k, pos, 1e6), synth.rope(q, pos[None].repeat(4, 0), 1e4))
    np.testing.assert_allclose(ek1, ek0, rtol=1e-12)
    np.testing.assert_allclose(eq1, eq0, rtol=1e-12)
    # a pairing of (i, i + d/2) instead of (2i, 2i+1) would not be invariant:
    pr = lambda x: (x[..., :64] ** 2 + x[..., 64:] ** 2).reshape(-1, 64).mean(0)
    assert not np.allclose(pr(synth.rope(k, pos, 1e6)), pr(k), rtol=1e-3)


def test_expected_energy_matches_generator_scale():
    w = synth.reduced(synth.WORKLOADS[1], t_cal=20000)
    kc, qc = synth.calibration(w, 0, 0)
    sq, sk = synth.block_sigmas(w, 0, 0)
    ek, eq = energy.block_energy(kc, qc)
    np.testing.assert_allclose(ek, 2 * sk ** 2, rtol=0.05)
    np.testing.assert_allclose(eq, 2 * sq ** 2, rtol=0.05)


def test_scores_and_sigma():
    ek = np.array([2.0, 0.0, 8.0, 0.5]); eq = np.array([1.0, 3.0, 0.25, 2.0])
    np.testing.assert_array_equal(energy.scores(ek, eq, "qk"), [2.0, 0.0, 2.0, 1.0])
    np.testing.assert_array_equal(energy.scores(ek, eq, "k"), ek)
    sigma, r = energy.sigma_hat(ek)
    assert sigma.dtype == np.float32
    np.testing.assert_array_equal(sigma, np.float32([1.0, 0.0, 2.0, 0.5]))
    np.testing.assert_array_equal(r, np.float32([1.0, 0.0, 0.5, 2.0]))


# ---------------------------------------------------------------- greedy
def _brute(s, U, bmax):
    best, arg, count = None, None, 0
    for b in itertools.product(range(bmax + 1), repeat=len(s)):
        if sum(b) != U or any(bi and si == 0 for bi, si in zip(b, s)):
            continue
        obj = allocate.objective(s, b)
        if best is None or obj < best - 1e-15 * best:
            best, arg, count = obj, b, 1
        elif abs(obj - best) <= 1e-15 * best:
            count += 1
    return best, arg, count


@pytest.mark.parametrize("seed", range(40))
def test_greedy_equals_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 6)); bmax = int(rng.integers(2, 5))
    U = int(rng.integers(1, min(12, n * bmax) + 1))
    s = np.exp(rng.uniform(-6, 6, n))
    if seed % 5 == 0:
        s = np.round(s)  # allow ties
        s[s == 0] = 1.0
    best, arg, count = _brute(list(s), U, bmax)
    got = allocate.greedy(s, U, bmax)
    assert got.sum() == U and got.max() <= bmax
    assert allocate.objective(s, got) == pytest.approx(best, rel=1e-12)
    if count == 1:
        assert tuple(got) == arg


@pytest.mark.parametrize("seed", range(10))
def test_exchange_certificate_and_monotone(seed):
    rng = np.random.default_rng(100 + seed)
    s = np.exp(rng.uniform(-10, 10, 64))
    U = 192
    b = allocate.greedy(s, U, 8)
    assert b.sum() == U
    gain_add = max(s[i] * 4.0 ** -b[i] for i in range(64) if b[i] < 8)
    gain_rm = min(s[j] * 4.0 ** -(b[j] - 1) for j in range(64) if b[j] > 0)
    assert gain_add <= gain_rm  # no single-bit move lowers the separable convex objective
    order = np.argsort(-s)
    assert np.all(np.diff(b[order]) <= 0)  # larger score -> at least as many bits


def test_water_filling_lower_bound():
    rng = np.random.default_rng(7)
    s = np.exp(rng.uniform(-4, 4, 16)); U, bmax = 40, 8
    b = allocate.greedy(s, U, bmax)
    # continuous relaxation: b_i = clip(theta + log2(s_i)/2, 0, bmax), sum = U (bisection on theta)
    lo, hi = -100.0, 100.0
    for _ in range(200):
        th = 0.5 * (lo + hi)
        tot = np.clip(th + 0.5 * np.log2(s), 0, bmax).sum()
        lo, hi = (th, hi) if tot < U else (lo, th)
    bc = np.clip(th + 0.5 * np.log2(s), 0, bmax)
    assert np.sum(s * 4.0 ** -bc) <= allocate.objective(s, b) * (1 + 1e-9)


def test_closed_form_cases():
    # equal scores: uniform, remainder to the lowest indices
    b = allocate.greedy(np.ones(6), 15, 8)
    np.testing.assert_array_equal(b, [3, 3, 3, 2, 2, 2])
    # s_i = 4^a_i: widths differ by exactly a_i (here all within range)
    a = np.array([0, 1, 3, 2, 0, 1])
    b = allocate.greedy(4.0 ** a, int(a.sum() + 6 * 2), 8)
    np.testing.assert_array_equal(b, a + 2)
    # zero score never receives bits; infeasible budget raises
    b = allocate.greedy([1.0, 0.0, 2.0], 10, 8)
    assert b[1] == 0 and b.sum() == 10
    with pytest.raises(allocate.BudgetError):
        allocate.greedy([1.0, 0.0, 2.0], 17, 8)


def test_ldexp_exact_ties_lowest_index():
    # s0 * 4^-1 == s1 exactly: the tie must go to block 0
    b = allocate.greedy([4.0, 1.0], 2, 8)
    np.testing.assert_array_equal(b, [2, 0])


# --- greedy under a tabulated rate (the realized Lloyd-Max D(b) instead of 4^-b) ---

def _lloyd_rate(bmax=8):
    from oracle import codebook
    return [1.0] + [codebook.codebook_mse(b) for b in range(1, bmax + 1)]


def test_realized_rate_is_convex_and_above_4_pow_minus_b():
    """The frozen tables' D(b) falls with shrinking steps (so the rate greedy is optimal) and sits
    above 4^-b by a factor that grows toward the Panter-Dite constant pi*sqrt(3)/2."""
    r = _lloyd_rate()
    gain = np.diff(r) * -1
    assert np.all(gain > 0) and np.all(np.diff(gain) < 0)
    ratio = [r[b] * 4.0 ** b for b in range(1, 9)]
    assert ratio[0] == pytest.approx(4 * (1 - 2 / np.pi), rel=1e-3)   # D(1) = 1 - 2/pi
    assert np.all(np.diff(ratio) > 0) and ratio[-1] < np.pi * np.sqrt(3) / 2


def _brute_rate(s, U, bmax, rate):
    best, arg, count = None, None, 0
    for b in itertools.product(range(bmax + 1), repeat=len(s)):
        if sum(b) != U or any(bi and si == 0 for bi, si in zip(b, s)):
            continue
        obj = allocate.objective_rate(s, b, rate)
        if best is None or obj < best - 1e-13 * best:
            best, arg, count = obj, b, 1
        elif abs(obj - best) <= 1e-13 * best:
            count += 1
    return best, arg, count


@pytest.mark.parametrize("seed", range(30))
def test_greedy_rate_equals_brute_force(seed):
    rng = np.random.default_rng(500 + seed)
    n = int(rng.integers(2, 6)); bmax = int(rng.integers(2, 5))
    U = int(rng.integers(1, min(12, n * bmax) + 1))
    s = np.exp(rng.uniform(-6, 6, n))
    rate = _lloyd_rate(bmax)
    best, arg, count = _brute_rate(list(s), U, bmax, rate)
    got = allocate.greedy_rate(s, U, rate, bmax)
    assert got.sum() == U and got.max() <= bmax
    assert allocate.objective_rate(s, got, rate) == pytest.approx(best, rel=1e-12)
    if count == 1:
        assert tuple(got) == arg


def test_greedy_rate_with_4_pow_minus_b_matches_greedy():
    """Under the idealized rate the gains are s_i 4^-b_i (3/4): the same ranking as greedy()."""
    rate = [4.0 ** -b for b in range(9)]
    for seed in range(20):
        rng = np.random.default_rng(900 + seed)
        s = np.exp(rng.uniform(-10, 10, 64))
        np.testing.assert_array_equal(allocate.greedy_rate(s, 192, rate), allocate.greedy(s, 192))


@pytest.mark.parametrize("seed", range(10))
def test_greedy_rate_beats_4_pow_minus_b_on_realized_distortion(seed):
    """On its own objective the rate greedy is never worse than the 4^-b allocation, and on
    heterogeneous heads the two allocations differ (the point of the option)."""
    rng = np.random.default_rng(300 + seed)
    s = np.exp(rng.uniform(-12, 12, 64))
    rate = _lloyd_rate()
    b_r = allocate.greedy_rate(s, 192, rate)
    b_4 = allocate.greedy(s, 192)
    assert allocate.objective_rate(s, b_r, rate) <= allocate.objective_rate(s, b_4, rate) * (1 + 1e-12)
    gain_add = max(s[i] * (rate[b_r[i]] - rate[b_r[i] + 1]) for i in range(64) if b_r[i] < 8)
    gain_rm = min(s[j] * (rate[b_r[j] - 1] - rate[b_r[j]]) for j in range(64) if b_r[j] > 0)
    assert gain_add <= gain_rm
    if seed == 0:
        assert not np.array_equal(b_r, b_4)


def test_greedy_rate_rejects_non_convex_rate():
    with pytest.raises(ValueError):
        allocate.greedy_rate([1.0, 2.0], 3, [1.0, 0.5, 0.4, 0.1], 3)   # steps 0.5, 0.1, 0.3
    with pytest.raises(ValueError):
        allocate.greedy_rate([1.0, 2.0], 3, [1.0, 0.5, 0.5, 0.4], 3)   # a flat step
