"""Cache construction and decode for whole layers, composed from the oracle's steps.

`calibrate` (energy -> scores -> greedy widths, sigma), `build_layer` (quantize every cached
token of every (batch, kv head) and lay the bytes out exactly as the GPU cache buffers) and
`decode_layer` (unpack -> dequantize -> fp64 attention for every query head).

Recent fp16 buffer (abstract: an fp16 recent-key buffer is an option the method can run
without; LogQuant summary, Method 2: a window of the most recent tokens kept at high
precision): with n_recent > 0, after N appended tokens the newest min(N, n_recent) stay in fp16
(rows rounded to fp16, ring slot = position mod n_recent) and the older ones are packed.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from . import allocate, attention, energy, layout, quantize
from .layout import TILE


@dataclasses.dataclass
class LayerMeta:
    bits: np.ndarray     # [Hkv, 64] int
    sigma: np.ndarray    # [Hkv, 64] fp32
    r: np.ndarray        # [Hkv, 64] fp32
    scores: np.ndarray   # [Hkv, 64] fp64


def calibrate(k_cals, q_cals, budget_units: int, b_max: int = 8, mode: str = "qk") -> LayerMeta:
    """k_cals[h] [T, d], q_cals[h] [g, T, d] for each kv head h."""
    bits, sig, rr, sc = [], [], [], []
    for kc, qc in zip(k_cals, q_cals):
        ek, eq = energy.block_energy(kc, qc)
        s = energy.scores(ek, eq, mode)
        sigma, r = energy.sigma_hat(ek)
        s = np.where(sigma > 0, s, 0.0)  # a dead block (sigma == 0) gets no bits
        bits.append(allocate.greedy(s, budget_units, b_max))
        sig.append(sigma); rr.append(r); sc.append(s)
    return LayerMeta(np.array(bits), np.array(sig), np.array(rr), np.array(sc))


@dataclasses.dataclass
class LayerCache:
    """Arrays mirror the GPU buffers of one layer byte for byte ([B][Hkv] leading dims)."""
    k_mode: str
    v_mode: str
    n_packed: int
    k_codes: np.ndarray   # uint8 [B, Hkv, n_tiles, tile_bytes]
    k_scale: np.ndarray   # fp16 [B, Hkv, n_cap] or [B, Hkv, n_cap, d/k_group]
    k_zero: np.ndarray | None
    v_codes: np.ndarray   # uint8 [B, Hkv, n_tiles, 1024*v_bits]
    v_scale: np.ndarray   # fp16 [B, Hkv, n_cap]
    v_zero: np.ndarray | None
    recent_k: np.ndarray | None  # fp16 [B, Hkv, n_recent, d]
    recent_v: np.ndarray | None
    n_recent_valid: int
    v_bits: int
    k_bits: int
    k_group: int
    meta: LayerMeta | None
    k_rot: np.ndarray | None = None   # +-1 [Hkv, d]: affine keys stored rotated (y = H (s * k) / 16)
    v_rot: np.ndarray | None = None   # +-1 [Hkv, d]: values stored rotated (y = H (s * v) / 16)


def build_layer(k_rows, v_rows, *, k_mode: str, v_mode: str, v_bits: int, n_cap: int,
                meta: LayerMeta | None = None, k_bits: int = 4, k_group: int = 32,
                n_recent: int = 0, k_rot=None, v_rot=None) -> LayerCache:
    """k_rows, v_rows: float32 [B, Hkv, N, d] (dtype-exact values), all N tokens appended.
    k_rot: optional +-1 signs [Hkv, d]; affine keys are then rotated before quantization (the
    fp16 recent buffer keeps the rows as they came).  v_rot: optional +-1 signs [Hkv, d]; values
    are then rotated the same way before quantization, and decode_layer undoes the rotation once
    on the output (caches without an fp16 recent buffer only: its rows would sit in the other
    space)."""
    if k_rot is not None and k_mode != "affine":
        raise ValueError("the key rotation applies to affine keys")
    if v_rot is not None and n_recent:
        raise ValueError("the value rotation applies to caches without an fp16 recent buffer")
    k_rows = np.asarray(k_rows, np.float32)
    v_rows = np.asarray(v_rows, np.float32)
    B, H, N, d = k_rows.shape
    n_rec = min(N, n_recent)
    n_packed = N - n_rec
    n_tiles = (n_cap + TILE - 1) // TILE
    if k_mode == "gtq":
        R = layout.k_gtq_dwords(int(meta.bits[0].sum()))
        k_scale = np.zeros((B, H, n_cap), np.float16)
        k_zero = None
    else:
        R = k_bits * d // 32
        k_scale = np.zeros((B, H, n_cap, d // k_group), np.float16)
        k_zero = np.zeros_like(k_scale)
    k_codes = np.zeros((B, H, n_tiles, TILE * R * 4), np.uint8)
    v_codes = np.zeros((B, H, n_tiles, 1024 * v_bits), np.uint8)
    v_scale = np.zeros((B, H, n_cap), np.float16)
    v_zero = np.zeros_like(v_scale) if v_mode == "affine" else None
    recent_k = recent_v = None
    if n_recent:
        recent_k = np.zeros((B, H, n_recent, d), np.float16)
        recent_v = np.zeros_like(recent_k)
    for b in range(B):
        for h in range(H):
            xk = k_rows[b, h, :n_packed]
            xv = v_rows[b, h, :n_packed]
            if v_rot is not None:
                xv = quantize.hadamard_rotate_f32(xv, v_rot[h])
            if k_mode == "gtq":
                codes, S = quantize.quantize_k_gtq(xk, meta.sigma[h], meta.r[h], meta.bits[h])
                words = layout.k_gtq_words(codes, meta.bits[h])
                k_scale[b, h, :n_packed] = S
            else:
                if k_rot is not None:
                    xk = quantize.hadamard_rotate_f32(xk, k_rot[h])
                codes, sc, zr = quantize.quantize_affine(xk, k_bits, k_group)
                words = layout.k_affine_words(codes, k_bits)
                k_scale[b, h, :n_packed] = sc
                k_zero[b, h, :n_packed] = zr
            k_codes[b, h] = layout.tile_records(words, n_tiles)
            if v_mode == "codebook":
                vc, S = quantize.quantize_v(xv, v_bits)
                v_scale[b, h, :n_packed] = S
            else:
                vc, sc, zr = quantize.quantize_affine(xv, v_bits, 128)
                v_scale[b, h, :n_packed] = sc[:, 0]
                v_zero[b, h, :n_packed] = zr[:, 0]
            v_codes[b, h] = layout.v_tiles(vc, v_bits, n_tiles)
            for pos in range(n_packed, N):
                recent_k[b, h, pos % n_recent] = k_rows[b, h, pos].astype(np.float16)
                recent_v[b, h, pos % n_recent] = v_rows[b, h, pos].astype(np.float16)
    return LayerCache(k_mode, v_mode, n_packed, k_codes, k_scale, k_zero, v_codes, v_scale, v_zero,
                      recent_k, recent_v, n_rec, v_bits, k_bits, k_group, meta,
                      None if k_rot is None else np.asarray(k_rot, np.float64),
                      None if v_rot is None else np.asarray(v_rot, np.float64))


def dequant_head(c: LayerCache, b: int, h: int):
    """(K_hat, V_hat) float64 [n_packed + n_recent_valid, d] for one (batch, kv head)."""
    n = c.n_packed
    n_tiles = c.k_codes.shape[2]
    if c.k_mode == "gtq":
        bits = c.meta.bits[h]
        R = layout.k_gtq_dwords(int(bits.sum()))
        codes = layout.k_gtq_codes(layout.untile_records(c.k_codes[b, h], n, R), bits)
        K = attention.dequant_k_gtq(codes, c.k_scale[b, h, :n], c.meta.sigma[h], bits)
    else:
        R = c.k_bits * 128 // 32
        codes = layout.k_affine_codes(layout.untile_records(c.k_codes[b, h], n, R), c.k_bits)
        K = attention.dequant_affine(codes, c.k_scale[b, h, :n], c.k_zero[b, h, :n], c.k_group)
        if c.k_rot is not None:
            K = attention.unrotate_keys(K, c.k_rot[h])   # back to the original key space, exactly
    vc = layout.v_codes(c.v_codes[b, h], c.v_bits, n)
    if c.v_mode == "codebook":
        V = attention.dequant_codebook(vc, c.v_scale[b, h, :n], c.v_bits)
    else:
        V = attention.dequant_affine(vc, c.v_scale[b, h, :n, None], c.v_zero[b, h, :n, None], 128)
    if c.n_recent_valid:
        rk = c.recent_k[b, h, :c.n_recent_valid].astype(np.float64)
        rv = c.recent_v[b, h, :c.n_recent_valid].astype(np.float64)
        K = np.concatenate([K, rk])
        V = np.concatenate([V, rv])
    return K, V


def decode_layer(c: LayerCache, q) -> np.ndarray:
    """q [B, Hq, d] (any float dtype) -> out float64 [B, Hq, d]."""
    q = np.asarray(q, np.float64)
    B, Hq, d = q.shape
    H = c.k_codes.shape[1]
    g = Hq // H
    out = np.zeros((B, Hq, d))
    for b in range(B):
        for h in range(H):
            K, V = dequant_head(c, b, h)
            o = attention.attend(q[b, h * g:(h + 1) * g], K, V)
            if c.v_rot is not None:   # V holds rotated values: undo the rotation once, on the output
                o = attention.unrotate_output(o, c.v_rot[h])
            out[b, h * g:(h + 1) * g] = o
    return out


def fp16_decode(k16, v16, q) -> np.ndarray:
    """Unquantized comparator: k16, v16 fp16 [B, Hkv, N, d]; q [B, Hq, d] -> float64 out."""
    k16 = np.asarray(k16, np.float16)
    v16 = np.asarray(v16, np.float16)
    q = np.asarray(q, np.float64)
    B, H, N, d = k16.shape
    g = q.shape[1] // H
    out = np.zeros(q.shape)
    for b in range(B):
        for h in range(H):
            out[b, h * g:(h + 1) * g] = attention.attend(
                q[b, h * g:(h + 1) * g], k16[b, h].astype(np.float64), v16[b, h].astype(np.float64))
    return out
