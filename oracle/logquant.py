"""LogQuant's log-based filter: which tokens stay at high precision as the context grows.

Test infrastructure only (the oracle): the library never imports it.

The LogQuant summary (Method 2) keeps a base window of W tokens: a reserved window of at most
3W high-precision tokens; when new tokens arrive at that limit, the density of the earlier part
is halved at regular intervals, which takes its count from 2W to W before new tokens refill
the window.  Repeated, the survivors of older windows thin out geometrically with distance
(spacings 1, 2, 4, ... toward the past), the log-distributed selection the summary describes.
Tokens that leave the high-precision set are quantized, not evicted (Method 3), and the order
of tokens does not matter to attention (Method 4).

Readings (the passage is garbled between 2W and 3W and names no parity):
- the high-precision set H never exceeds 3W tokens;
- when a token arrives and |H| = 3W, the 2W oldest members of H (by position) are halved:
  the 1st, 3rd, 5th, ... oldest stay, the 2nd, 4th, ... leave H for the low-bit store, oldest
  first; then the new token joins H;
- so the oldest token ever seen stays at high precision (it is always the first of its pair).
"""
from __future__ import annotations


def select(n_tokens: int, W: int):
    """Append positions 0 .. n_tokens-1 one at a time.  Returns (hp, quantized): hp = the
    high-precision positions in ascending order; quantized = the positions in the order they
    left hp (each thinning lists its leavers oldest first)."""
    if W < 1:
        raise ValueError("W must be at least 1")
    hp: list[int] = []
    quantized: list[int] = []
    for p in range(n_tokens):
        if len(hp) == 3 * W:
            older, recent = hp[:2 * W], hp[2 * W:]
            quantized.extend(older[1::2])
            hp = older[0::2] + recent
        hp.append(p)
    return hp, quantized
