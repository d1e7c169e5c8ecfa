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
Tile of K records: split each record into chunks of 4 dwords (the last may be shorter); chunk
c of all 64 tokens occupies one region starting at byte c*1024, token t's chunk at
t * (chunk dwords) * 4 inside the region.

V tile (b bits, codebook or affine): 32 token pairs (2p, 2p+1) x 8 dim groups of 16 dims x
b dwords, in that order (pair-major).  Within the b dwords of (pair p, group G), dim 16G+j
has a 2b-bit field at bit 2b*j: low b bits = code of token 2p, high b bits = code of 2p+1.
A token that does not exist contributes zero bits.

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


def _chunks(R: int):
    return [(c * 1024, min(4, R - 4 * c)) for c in range((R + 3) // 4)]


def tile_records(words: np.ndarray, n_tiles: int) -> np.ndarray:
    """records [n, R] -> tiles uint8 [n_tiles, 64*R*4] in the chunked token-minor layout."""
    n, R = words.shape
    padded = np.zeros((n_tiles * TILE, R), np.uint32)
    padded[:n] = words
    padded = padded.reshape(n_tiles, TILE, R)
    out = np.zeros((n_tiles, TILE * R), np.uint32)
    for c, (off, cs) in enumerate(_chunks(R)):
        base = off // 4
        out[:, base:base + TILE * cs] = padded[:, :, 4 * c:4 * c + cs].reshape(n_tiles, TILE * cs)
    return out.view(np.uint8).reshape(n_tiles, TILE * R * 4)


def untile_records(tiles: np.ndarray, n: int, R: int) -> np.ndarray:
    n_tiles = tiles.shape[0]
    t32 = np.ascontiguousarray(tiles).view(np.uint32).reshape(n_tiles, TILE * R)
    words = np.zeros((n_tiles, TILE, R), np.uint32)
    for c, (off, cs) in enumerate(_chunks(R)):
        base = off // 4
        words[:, :, 4 * c:4 * c + cs] = t32[:, base:base + TILE * cs].reshape(n_tiles, TILE, cs)
    return words.reshape(n_tiles * TILE, R)[:n]


def v_tiles(codes: np.ndarray, b: int, n_tiles: int) -> np.ndarray:
    """codes [n, 128] -> tiles uint8 [n_tiles, 1024*b] in the pair-major layout."""
    n, d = codes.shape
    assert d == 128
    npairs = n_tiles * TILE // 2
    even = np.zeros((npairs, d), np.int64)
    odd = np.zeros((npairs, d), np.int64)
    even[: (n + 1) // 2] = codes[0::2]
    odd[: n // 2] = codes[1::2]
    words = np.zeros((npairs * 8, b), np.uint32)  # rows = (pair, group)
    for G in range(8):
        rows = slice(G, None, 8)
        sub = np.zeros((npairs, b), np.uint32)
        for j in range(16):
            dim = 16 * G + j
            field = even[:, dim] | (odd[:, dim] << b)
            _put(sub, 2 * b * j, 2 * b, field)
        words[rows] = sub
    return words.reshape(n_tiles, TILE // 2 * 8 * b).view(np.uint8).reshape(n_tiles, 1024 * b)


def v_codes(tiles: np.ndarray, b: int, n: int) -> np.ndarray:
    t32 = np.ascontiguousarray(tiles).view(np.uint32).reshape(-1, b)  # rows = (tile, pair, group)
    npairs = tiles.shape[0] * TILE // 2
    codes = np.zeros((2 * npairs, 128), np.int64)
    for G in range(8):
        sub = t32[G::8]
        for j in range(16):
            field = _get(sub, 2 * b * j, 2 * b)
            codes[0::2, 16 * G + j] = field & ((1 << b) - 1)
            codes[1::2, 16 * G + j] = field >> b
    return codes[:n]
