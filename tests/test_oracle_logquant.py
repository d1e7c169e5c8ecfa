"""Pins of the LogQuant selection oracle (oracle/logquant.py) to what the LogQuant summary
(Method 2) fixes: a 3W ceiling, halving of the older part at regular intervals from 2W to W, and
the resulting geometric thinning with distance.  Hand-worked example plus invariants."""
import pytest

from oracle import logquant as lq


def test_hand_worked_w4():
    # W = 4 (ceiling 12), worked by hand from the rule:
    #  p=12: older [0..7] -> keep 0 2 4 6, leave 1 3 5 7
    #  p=16: older [0 2 4 6 8 9 10 11] -> keep 0 4 8 10, leave 2 6 9 11
    #  p=20: older [0 4 8 10 12 13 14 15] -> keep 0 8 12 14, leave 4 10 13 15
    hp, q = lq.select(21, 4)
    assert hp == [0, 8, 12, 14, 16, 17, 18, 19, 20]
    assert q == [1, 3, 5, 7, 2, 6, 9, 11, 4, 10, 13, 15]


def test_below_the_ceiling_everything_stays():
    for W in (1, 2, 8):
        hp, q = lq.select(3 * W, W)
        assert hp == list(range(3 * W)) and q == []


@pytest.mark.parametrize("W", [1, 2, 3, 4, 8, 16])
def test_invariants(W):
    hp_prev = []
    for n in range(1, 40 * W):
        hp, q = lq.select(n, W)
        assert len(hp) <= 3 * W                                    # the reserved window
        assert sorted(hp) == hp and sorted(set(hp) | set(q)) == list(range(n))
        assert not set(hp) & set(q)                                # every token in exactly one store
        assert hp[-min(n, W + 1):] == list(range(n - min(n, W + 1), n))   # newest W + 1 always dense
        assert hp[0] == 0                                          # the first of every pair stays
        if len(hp_prev) == 3 * W:                                  # a thinning happened: 2W -> W
            assert len(hp) == 2 * W + 1
        hp_prev = hp


def test_spacing_doubles_toward_the_past():
    # The gaps between kept positions, read from the newest backward, never shrink (density falls
    # with distance, the summary's Method 2), and each is a power of two, the halvings it names;
    # the oldest gap excepted, since the first token, always the first of its pair, never leaves.
    W = 8
    for n in range(6 * W, 60 * W, 7):
        hp, _ = lq.select(n, W)
        gaps = [b - a for a, b in zip(hp, hp[1:])][::-1]
        assert all(g & (g - 1) == 0 for g in gaps[:-1]), gaps
        assert all(x <= y for x, y in zip(gaps, gaps[1:])), (n, gaps)
        assert max(gaps[:-1]) <= 2 ** (n // W)                  # bounded by the number of halvings


def test_high_precision_count_grows_logarithmically():
    # the count stays within [2W + 1, 3W] once the ceiling is reached, however long the context
    W = 4
    for n in (3 * W + 1, 100, 1000, 5000):
        hp, q = lq.select(n, W)
        assert 2 * W + 1 <= len(hp) <= 3 * W and len(hp) + len(q) == n
