"""Greedy integer bit allocation over RoPE blocks (Block-GTQ).

Block-GTQ (abstract; review §3, Figure 1) gives integer widths per RoPE block, per layer
and KV head, greedily by marginal gain, with the TQ-MSE distortion rate 4^-b ranking the
gains.  With block distortion s_i * 4^-b_i, adding one bit to block i lowers the objective
by s_i * 4^-b_i * 3/4, so each step picks the block with the largest s_i * 4^-b_i.

Readings: all widths start at 0; a step may pick only blocks with b_i < b_max and s_i > 0
(a block with zero score gets no bits); ties go to the lowest block index; the key
s_i * 4^-b_i is formed exactly with ldexp.  A budget the candidates cannot absorb is an
error.  Budget unit = one bit per coordinate of one block (a block has 2 coordinates), so
the K record holds 2 * U bits per token (U = 128 for "K2", 192 for "K3").
"""
from __future__ import annotations

import math

import numpy as np


class BudgetError(ValueError):
    pass


def greedy(s, budget_units: int, b_max: int = 8, b_min: int = 0) -> np.ndarray:
    s = [float(x) for x in s]
    n = len(s)
    b = [0] * n
    spent = 0
    if b_min:
        for i in range(n):
            if s[i] > 0:
                b[i] = b_min
                spent += b_min
    if spent > budget_units:
        raise BudgetError("b_min exceeds budget")
    for _ in range(budget_units - spent):
        best, best_key = -1, None
        for i in range(n):
            if b[i] < b_max and s[i] > 0:
                key = math.ldexp(s[i], -2 * b[i])
                if best_key is None or key > best_key:
                    best, best_key = i, key
        if best < 0:
            raise BudgetError("budget exceeds what the live blocks can hold")
        b[best] += 1
    return np.array(b, dtype=np.int64)


def objective(s, bits) -> float:
    """Modelled key distortion sum_i s_i * 4^-b_i."""
    return float(sum(math.ldexp(float(si), -2 * int(bi)) for si, bi in zip(s, bits)))


def greedy_rate(s, budget_units: int, rate, b_max: int = 8, b_min: int = 0) -> np.ndarray:
    """Greedy widths under a tabulated distortion-rate curve instead of the idealized 4^-b.

    The review (§3) ranks marginal gains with the TQ-MSE rate 4^-b; a real scalar quantizer
    reaches D(b) (the frozen Lloyd-Max table: D(1..3) ~ 0.363, 0.117, 0.0346), whose ratios
    D(b)/D(b+1) approach 4 only for wide codes.  With block distortion s_i * D(b_i), adding a bit
    to block i lowers the objective by s_i * (D(b_i) - D(b_i + 1)); each step picks the largest
    such gain (ties: lowest index), among blocks with b_i < b_max and s_i > 0.  rate[b] = D(b)
    for b = 0..b_max must fall with non-increasing steps (a convex curve), the condition under
    which this greedy is optimal for the separable objective sum_i s_i D(b_i).
    """
    s = [float(x) for x in s]
    rate = [float(x) for x in rate]
    if len(rate) < b_max + 1:
        raise ValueError("rate needs b_max + 1 entries")
    gain = [rate[b] - rate[b + 1] for b in range(b_max)]
    if any(not g > 0 for g in gain) or any(gain[b + 1] > gain[b] for b in range(b_max - 1)):
        raise ValueError("rate must decrease with non-increasing steps")
    n = len(s)
    b = [0] * n
    spent = 0
    if b_min:
        for i in range(n):
            if s[i] > 0:
                b[i] = b_min
                spent += b_min
    if spent > budget_units:
        raise BudgetError("b_min exceeds budget")
    for _ in range(budget_units - spent):
        best, best_key = -1, None
        for i in range(n):
            if b[i] < b_max and s[i] > 0:
                key = s[i] * gain[b[i]]
                if best_key is None or key > best_key:
                    best, best_key = i, key
        if best < 0:
            raise BudgetError("budget exceeds what the live blocks can hold")
        b[best] += 1
    return np.array(b, dtype=np.int64)


def objective_rate(s, bits, rate) -> float:
    """Modelled key distortion sum_i s_i * D(b_i) under a tabulated rate."""
    return float(sum(float(si) * float(rate[int(bi)]) for si, bi in zip(s, bits)))
