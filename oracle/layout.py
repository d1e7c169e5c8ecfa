"""Byte layout of the packed KV cache (the oracle's own packer and unpacker).

The pages fix no format, only that attention reads the compressed K/V directly without an
fp16 copy (review §1 Packed-Cache, Figure 2; abstract).  The layout below is this
library's contract; the GPU writes exactly these bytes.

Tokens are grouped in tiles of TILE = 64 consecutive positions of one (batch, kv head).

K record (Block-GTQ): a little-endian bit stream of R = 2U/32 dwords per token (bit p is bit
p%32 of dword p/32).  Blocks appear in "block order": width descending, ties by ascending
block index, width-0 blocks omitted; block i of width w puts code(2i) at the next w bits and
code(2i+1) at the w bits after it.
K record (affine, b bits): coordinate j at bits [b*j, b*j + b).
Tile of K records (R dwords per token): dword-major, token-minor — dword k of token t at byte
(k*64 + t)*4, so the k-th dword of all 64 tokens is one contiguous 256-byte row.

V tile (b bits, codebook or affine): 16 token quads (4q .. 4q+3) x 16 dim groups of 8 dims x
b dwords, in that order (quad-major).  The b dwords of (quad q, group G) hold 16 fields of 2b
bits, field f at bit 2b*f: token pair 2q + f//8 (tokens 4q + 2(f//8) and the next one), dim
8G + f%8; low b bits = code of the even token, high b bits = code of the odd token.  A token
that does not exist contributes zero bits.

Scales: fp16 arrays indexed [token] (codebook K/V) or [token][group] (affine), one per
(batch, kv head), outside the tiles.
"""
from __future__ import annotations

import numpy as np

TILE = 64


def block_order(bits) -> np.ndarray:
    bits = np.asarray(bits)
    idx = [i for i in range(len(bits)) if bits[i] > 0]
    return np.array(sorted(idx, key=lambda i: (-int(bits[i]), i)), dtype=np.int64)


def k_gtq_dwords(budget_units: int) -> int:
    if (2 * budget_units) % 32:
        raise ValueError("2*U must be a multiple of 32")
    return 2 * budget_units // 32


def _put(words: np.ndarray, pos: int, width: int, vals: np.ndarray) -> None:
    """OR `width`-bit values into the bit stream of every row at bit position pos."""
    v = vals.astype(np.uint64) & np.uint64((1 << width) - 1)
    w, s = pos // 32, pos % 32
    shifted = v << np.uint64(s)
    words[:, w] |= (shifted & np.uint64(0xFFFFFFFF)).astype(np.uint32)
    if s + width > 32:
        words[:, w + 1] |= (shifted >> np.uint64(32)).astype(np.uint32)


def _get(words: np.ndarray, pos: int, width: int) -> np.ndarray:
    w, s = pos // 32, pos % 32
    v = words[:, w].astype(np.uint64) >> np.uint64(s)
    if s + width > 32:
        v |= words[:, w + 1].astype(np.uint64) << np.uint64(32 - s)
    return (v & np.uint64((1 << width) - 1)).astype(np.int64)


def k_gtq_words(codes: np.ndarray, bits) -> np.ndarray:
    """codes [n, d] -> records [n, R] uint32."""
    bits = np.asarray(bits)
    n = codes.shape[0]
    R = k_gtq_dwords(int(bits.sum()))
    words = np.zeros((n, R), np.uint32)
    pos = 0
    for i in block_order(bits):
        w = int(bits[i])
        _put(words, pos, w, codes[:, 2 * i])
        _put(words, pos + w, w, codes[:, 2 * i + 1])
        pos += 2 * w
    assert pos == 32 * R
    return words


def k_gtq_codes(words: np.ndarray, bits) -> np.ndarray:
    bits = np.asarray(bits)
    n = words.shape[0]
    codes = np.zeros((n, 2 * len(bits)), np.int64)
    pos = 0
    for i in block_order(bits):
        w = int(bits[i])
        codes[:, 2 * i] = _get(words, pos, w)
        codes[:, 2 * i + 1] = _get(words, pos + w, w)
        pos += 2 * w
    return codes


def k_affine_words(codes: np.ndarray, b: int) -> np.ndarray:
    n, d = codes.shape
    words = np.zeros((n, b * d // 32), np.uint32)
    for j in range(d):
        _put(words, b * j, b, codes[:, j])
    return words


def k_affine_codes(words: np.ndarray, b: int, d: int = 128) -> np.ndarray:
    return np.stack([_get(words, b * j, b) for j in range(d)], axis=1)


def tile_records(words: np.ndarray, n_tiles: int) -> np.ndarray:
    """records [n, R] -> tiles uint8 [n_tiles, 64*R*4], dword-major token-minor."""
    n, R = words.shape
    padded = np.zeros((n_tiles * TILE, R), np.uint32)
    padded[:n] = words
    out = padded.reshape(n_tiles, TILE, R).transpose(0, 2, 1).copy()  # [tile, k, t]
    return out.view(np.uint8).reshape(n_tiles, TILE * R * 4)


def untile_records(tiles: np.ndarray, n: int, R: int) -> np.ndarray:
    n_tiles = tiles.shape[0]
    t32 = np.ascontiguousarray(tiles).view(np.uint32).reshape(n_tiles, R, TILE)
    return t32.transpose(0, 2, 1).reshape(n_tiles * TILE, R)[:n]


def v_tiles(codes: np.ndarray, b: int, n_tiles: int) -> np.ndarray:
    """codes [n, 128] -> tiles uint8 [n_tiles, 1024*b] in the quad-major layout."""
    n, d = codes.shape
    assert d == 128
    full = np.zeros((n_tiles * TILE, d), np.int64)
    full[:n] = codes
    quads = full.reshape(n_tiles * TILE // 4, 4, d)          # [quad, token in quad, dim]
    rows = np.zeros((quads.shape[0], 16, b), np.uint32)       # [quad, group, dword]
    for G in range(16):
        sub = np.zeros((quads.shape[0], b), np.uint32)
        for f in range(16):
            pr, dim = f // 8, 8 * G + f % 8
            field = quads[:, 2 * pr, dim] | (quads[:, 2 * pr + 1, dim] << b)
            _put(sub, 2 * b * f, 2 * b, field)
        rows[:, G] = sub
    return rows.reshape(n_tiles, 1024 * b // 4).view(np.uint8).reshape(n_tiles, 1024 * b)


def v_codes(tiles: np.ndarray, b: int, n: int) -> np.ndarray:
    n_tiles = tiles.shape[0]
    rows = np.ascontiguousarray(tiles).view(np.uint32).reshape(n_tiles * TILE // 4, 16, b)
    quads = np.zeros((rows.shape[0], 4, 128), np.int64)
    for G in range(16):
        for f in range(16):
            pr, dim = f // 8, 8 * G + f % 8
            field = _get(rows[:, G], 2 * b * f, 2 * b)
            quads[:, 2 * pr, dim] = field & ((1 << b) - 1)
            quads[:, 2 * pr + 1, dim] = field >> b
    return quads.reshape(-1, 128)[:n]
