"""Label-free RoPE-block energy scores from calibration data.

Block-GTQ (abstract; review §3) computes, for each layer and KV head, an energy score per
RoPE block from calibration data, higher energy meaning more sensitivity of the q·k
logits.  The formula is not printed.  Reading used here (documented as a reading):

  E_k[i] = mean over calibration tokens of ||k_(2i, 2i+1)||^2
  E_q[i] = mean over calibration tokens and the g query heads of the group of ||q_(2i, 2i+1)||^2
  s_i    = E_q[i] * E_k[i]            (mode "qk", default)
  s_i    = E_k[i]                     (mode "k", keys only)

Under a uniform RoPE phase and independent q, k, the expected squared logit error of block i
is proportional to E_q[i] times the key error energy, which the 4^-b rate makes E_k[i]*4^-b_i.
Block norms are RoPE-invariant, so post-RoPE calibration rows can be used directly.
The per-block key scale used by the quantizer is sigma_i = sqrt(E_k[i] / 2) (per-coordinate
RMS), stored in fp32, with r_i = fp32(1 / sigma_i) (0 for a dead block).
"""
from __future__ import annotations

import numpy as np


def block_energy(k_cal: np.ndarray, q_cal: np.ndarray):
    """k_cal [T, d], q_cal [g, T, d] (any float dtype) -> (E_k[d/2], E_q[d/2]) float64."""
    k = np.asarray(k_cal, dtype=np.float64)
    q = np.asarray(q_cal, dtype=np.float64)
    if q.ndim == 2:
        q = q[None]
    T, d = k.shape
    ek = np.zeros(d // 2)
    eq = np.zeros(d // 2)
    for i in range(d // 2):
        ek[i] = np.mean(k[:, 2 * i] ** 2 + k[:, 2 * i + 1] ** 2)
        eq[i] = np.mean(q[:, :, 2 * i] ** 2 + q[:, :, 2 * i + 1] ** 2)
    return ek, eq


def scores(ek: np.ndarray, eq: np.ndarray, mode: str = "qk") -> np.ndarray:
    if mode == "qk":
        return np.asarray(eq, np.float64) * np.asarray(ek, np.float64)
    if mode == "k":
        return np.asarray(ek, np.float64).copy()
    raise ValueError(mode)


def sigma_hat(ek: np.ndarray):
    """(sigma fp32 [nb], r = fp32(1/sigma) [nb]); r = 0 where sigma == 0."""
    sigma = np.sqrt(np.asarray(ek, np.float64) / 2.0).astype(np.float32)
    r = np.zeros_like(sigma)
    live = sigma > 0
    r[live] = np.float32(1.0) / sigma[live]  # fp32 division, correctly rounded
    return sigma, r
