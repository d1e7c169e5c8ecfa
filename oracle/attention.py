"""Dequantization and float64 decode attention over the packed cache.

Packed-cache serving (review §1 Packed-Cache, Figure 2; abstract) computes attention from
the compressed K/V.  The oracle dequantizes exactly in float64 and applies single-query
softmax attention with scale 1/sqrt(d), no mask:
  z_t = q . k_hat_t / sqrt(d),  p_t = exp(z_t - max z),  o = sum_t p_t v_hat_t / sum_t p_t.
Tokens of an fp16 recent buffer are concatenated with the packed tokens; their order does
not matter (LogQuant summary, Method 4: A·V = A_P·V_P).

Split-K: a split over a token subset returns (m, l, o_unnormalised) with m = max z,
l = sum exp(z - m), o = sum exp(z - m) v; `merge` combines splits by rescaling to the
global max (log-sum-exp), which equals one pass over all tokens.
"""
from __future__ import annotations

import numpy as np

from .codebook import codebook


def dequant_k_gtq(codes: np.ndarray, S: np.ndarray, sigma: np.ndarray, bits) -> np.ndarray:
    n, d = codes.shape
    out = np.zeros((n, d))
    S64 = np.asarray(S, np.float16).astype(np.float64)
    for i in range(d // 2):
        b = int(bits[i])
        if b == 0:
            continue
        if b == 16:  # oracle-only passthrough: the code is an fp16 bit pattern
            pair = codes[:, 2 * i:2 * i + 2].astype(np.uint16).view(np.float16)
            out[:, 2 * i:2 * i + 2] = pair.astype(np.float64)
            continue
        c = codebook(b)[0].astype(np.float64)
        s = float(np.float32(sigma[i]))
        out[:, 2 * i] = S64 * s * c[codes[:, 2 * i]]
        out[:, 2 * i + 1] = S64 * s * c[codes[:, 2 * i + 1]]
    return out


def dequant_codebook(codes: np.ndarray, S: np.ndarray, b: int) -> np.ndarray:
    c = codebook(b)[0].astype(np.float64)
    return np.asarray(S, np.float16).astype(np.float64)[:, None] * c[codes]


def dequant_affine(codes: np.ndarray, scale: np.ndarray, zero: np.ndarray, group: int) -> np.ndarray:
    n, d = codes.shape
    s = np.repeat(np.asarray(scale, np.float16).astype(np.float64), group, axis=1)
    z = np.repeat(np.asarray(zero, np.float16).astype(np.float64), group, axis=1)
    return s * codes + z


def partial(q: np.ndarray, K: np.ndarray, V: np.ndarray):
    """q [g, d], K, V [n, d] (float64) -> (m [g], l [g], o_unnorm [g, d])."""
    q = np.asarray(q, np.float64)
    d = q.shape[-1]
    z = (q @ np.asarray(K, np.float64).T) / np.sqrt(d)  # [g, n]
    m = z.max(axis=1)
    p = np.exp(z - m[:, None])
    return m, p.sum(axis=1), p @ np.asarray(V, np.float64)


def merge(parts):
    """Combine split partials [(m, l, o_unnorm), ...] into the normalised output [g, d]."""
    M = np.max(np.stack([m for m, _, _ in parts]), axis=0)
    L = sum(l * np.exp(m - M) for m, l, _ in parts)
    O = sum(o * np.exp(m - M)[:, None] for m, _, o in parts)
    return O / L[:, None]


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    m, l, o = partial(q, K, V)
    return o / l[:, None]


def hadamard_matrix(d: int = 128) -> np.ndarray:
    """Sylvester Hadamard matrix: H[i, j] = (-1)^popcount(i & j)."""
    i = np.arange(d)
    par = np.array([[bin(a & b).count("1") & 1 for b in i] for a in i])
    return np.where(par == 0, 1.0, -1.0)


def unrotate_keys(k_rot: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """Inverse of the key rotation y = H (s * x) / 16 in float64: x = s * (H y) / 8 (H H = 128 I)."""
    H = hadamard_matrix(k_rot.shape[-1])
    return np.asarray(signs, np.float64) * (np.asarray(k_rot, np.float64) @ H.T) / 8.0


def unrotate_output(o_rot: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """Undo the value rotation once, on the attention output ("Quantize What Counts" summary,
    Results, rotation integration: values rotated before quantization).  With values stored as
    y_t = H (s * v_t) / 16, the output over them is o' = sum_t p_t y_t / sum_t p_t = H (s * o) / 16
    by linearity, so o = s * (H o') / 8 (H H = 128 I), in float64."""
    H = hadamard_matrix(o_rot.shape[-1])
    return np.asarray(signs, np.float64) * (np.asarray(o_rot, np.float64) @ H.T) / 8.0
