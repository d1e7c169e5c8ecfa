"""Per-token quantization of cached K/V rows into integer codes plus fp16 scales.

Block-GTQ keys (abstract; review §1 TQ-MSE, §3): each RoPE block i gets b_i bits per
coordinate.  Reading used for the TQ-MSE step (the pages give no formula): whiten each
coordinate by its block's calibration scale, normalise the token by its RMS, and quantize
each coordinate with the Lloyd-Max N(0,1) table of its block's width.  No cross-block random
rotation (it would mix the blocks the allocation separates).  Values use the same quantizer
with sigma = 1 and one width for every coordinate ("uniform" width, abstract).

The float32 arithmetic is specified one IEEE operation at a time so a GPU can reproduce the
integer outputs exactly:
  u_j  = x_j * r_i                  (r_i = fp32(1/sigma_i); r = 1 for values)
  acc  = ((0 + u_0*u_0) + u_1*u_1) + ...   sequential over j = 0..d-1, no FMA
  S    = fp16_rne( sqrt_f32( acc / d ) )   (one fp16 scale per token)
  t_i  = fp32( S * sigma_i )
  code = #{ m : x_j >= fp32(t_i * tau_{b,m}) }   (tau: the frozen fp32 thresholds)
Dequantization: x_hat_j = S * sigma_i * c_b[code_j] (exact in float64).

Affine groups (the "Quantize What Counts" summary: 4-bit keys with group 32, 2-bit values
with group 128; read as min/max affine groups along head_dim within each token):
  scale = fp16_rne( fp32(max - min) / (2^b - 1) ),  zero = fp16_rne(min)
  code  = clamp( rint_even( fp32(x - zero) / scale ), 0, 2^b - 1 ), code = 0 if scale == 0
  x_hat = scale * code + zero.
Inputs must be finite with |x| <= 65504 and produce finite scales; anything else is undefined.
"""
from __future__ import annotations

import numpy as np

from .codebook import codebook

F32 = np.float32
PASSTHROUGH = 16  # oracle-only width: store the fp16 value itself (unquantized check)


def rms_scale(x: np.ndarray, r_coord: np.ndarray) -> np.ndarray:
    """x [n, d] float32, r_coord [d] float32 -> S [n] float16 (sequential fp32 sum)."""
    x = np.asarray(x, F32)
    r_coord = np.asarray(r_coord, F32)
    n, d = x.shape
    acc = np.zeros(n, F32)
    for j in range(d):
        u = x[:, j] * r_coord[j]
        acc = acc + u * u
    ms = acc / F32(d)
    return np.sqrt(ms).astype(np.float16)


def tq_codes(x: np.ndarray, t: np.ndarray, b: int) -> np.ndarray:
    """Count of scaled thresholds at or below x.  x, t float32 [n] -> int64 [n]."""
    _, thr = codebook(b)
    x = np.asarray(x, F32)
    t = np.asarray(t, F32)
    out = np.empty(len(x), np.int64)
    step = max(1, (1 << 22) // len(thr))
    for s in range(0, len(x), step):
        theta = t[s:s + step, None] * thr[None, :]          # fp32 products
        out[s:s + step] = (x[s:s + step, None] >= theta).sum(axis=1)
    return out


def quantize_k_gtq(x: np.ndarray, sigma: np.ndarray, r: np.ndarray, bits: np.ndarray):
    """Keys [n, d] -> (codes [n, d] int64 (0 where the block width is 0), S [n] fp16)."""
    x = np.asarray(x, F32)
    sigma = np.asarray(sigma, F32)
    n, d = x.shape
    S = rms_scale(x, np.repeat(np.asarray(r, F32), 2))
    S32 = S.astype(F32)
    codes = np.zeros((n, d), np.int64)
    for i in range(d // 2):
        b = int(bits[i])
        if b == 0:
            continue
        if b == PASSTHROUGH:  # oracle-only: the code is the fp16 bit pattern of x
            codes[:, 2 * i:2 * i + 2] = x[:, 2 * i:2 * i + 2].astype(np.float16).view(np.uint16)
            continue
        t = S32 * sigma[i]
        codes[:, 2 * i] = tq_codes(x[:, 2 * i], t, b)
        codes[:, 2 * i + 1] = tq_codes(x[:, 2 * i + 1], t, b)
    return codes, S


def quantize_v(x: np.ndarray, b: int):
    """Values [n, d] -> (codes [n, d], S [n] fp16): uniform width b, sigma = 1."""
    x = np.asarray(x, F32)
    n, d = x.shape
    S = rms_scale(x, np.ones(d, F32))
    S32 = S.astype(F32)
    codes = np.zeros((n, d), np.int64)
    for j in range(d):
        codes[:, j] = tq_codes(x[:, j], S32, b)
    return codes, S


def quantize_affine(x: np.ndarray, b: int, group: int):
    """[n, d] -> (codes [n, d], scale fp16 [n, d/group], zero fp16 [n, d/group])."""
    x = np.asarray(x, F32)
    n, d = x.shape
    xg = x.reshape(n, d // group, group)
    mn = xg.min(axis=-1)
    mx = xg.max(axis=-1)
    scale16 = ((mx - mn) / F32(2 ** b - 1)).astype(np.float16)
    zero16 = mn.astype(np.float16)
    s32 = scale16.astype(F32)[..., None]
    z32 = zero16.astype(F32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = (xg - z32) / s32
    code = np.clip(np.rint(q), 0, 2 ** b - 1)
    code = np.where(s32 == 0, 0, code)
    return code.reshape(n, d).astype(np.int64), scale16, zero16


def hadamard_rotate_f32(x: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """Rotation of rows before quantization (affine keys, or values): y = H (s * x) / 16 in float32.

    The "Quantize What Counts" summary (Results, rotation integration) reports that rotating the
    keys alone, in the K4V2 setting, brings accuracy close to K4V4 (rotation spreads key outlier
    channels over a group), while rotating the values alone gives marginal or negative results; it
    names no rotation.
    Reading: a randomized Hadamard rotation, H the 128x128 Sylvester Hadamard matrix, s a
    caller-given +-1 sign per coordinate.  H (s * x) is computed by the fast transform with stages
    h = 1, 2, 4, ..., 64 in that order; at stage h each pair (j, j + h) with bit h of j clear
    becomes (a + b, a - b), one float32 addition or subtraction each; the final 1/16 is exact.
    """
    y = np.asarray(x, F32) * np.asarray(signs, F32)
    d = y.shape[-1]
    h = 1
    while h < d:
        y = y.copy()
        for i0 in range(0, d, 2 * h):
            a = y[..., i0:i0 + h].copy()
            b = y[..., i0 + h:i0 + 2 * h].copy()
            y[..., i0:i0 + h] = a + b
            y[..., i0 + h:i0 + 2 * h] = a - b
        h *= 2
    return (y * F32(1.0 / 16.0)).astype(F32)
