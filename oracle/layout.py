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

V tile (b bits, codebook or affine), "lane-stream" order: the tile is split into 64 streams of
4*b dwords, one per lane L = dd + 16*j (dd in 0..15, j in 0..3).  Stream L holds 64 fields of 2b
bits, field phi = (s*8 + db)*4 + m (s in 0..1, db in 0..7, m in 0..3) at bit 2b*phi: the codes
of dim 16*db + dd for the token pair (p, p + 32), p = 16*s + 4*j + m, code of p in the low b
bits.  Stream dword c sits at tile dword ((c // 4)*64 + L)*4 + c % 4, so a wave reads the tile
with b loads of 16 bytes per lane.

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


def _v_lane_fields(L: int):
    """(field index, token p, dim) of every field in lane L's stream."""
    dd, j = L % 16, L // 16
    out = []
    for s_ in range(2):
        for db in range(8):
            for m in range(4):
                out.append(((s_ * 8 + db) * 4 + m, 16 * s_ + 4 * j + m, 16 * db + dd))
    return out


def v_tiles(codes: np.ndarray, b: int, n_tiles: int) -> np.ndarray:
    """codes [n, 128] -> tiles uint8 [n_tiles, 1024*b] in the lane-stream layout."""
    n, d = codes.shape
    assert d == 128
    full = np.zeros((n_tiles * TILE, d), np.int64)
    full[:n] = codes
    tok = full.reshape(n_tiles, TILE, d)
    streams = np.zeros((n_tiles, 64, 4 * b), np.uint32)       # [tile, lane, stream dword]
    for L in range(64):
        for phi, p, dim in _v_lane_fields(L):
            field = tok[:, p, dim] | (tok[:, p + 32, dim] << b)
            _put(streams[:, L], 2 * b * phi, 2 * b, field)
    out = streams.reshape(n_tiles, 64, b, 4).transpose(0, 2, 1, 3)  # [tile, c // 4, lane, c % 4]
    return np.ascontiguousarray(out).view(np.uint8).reshape(n_tiles, 1024 * b)


def v_codes(tiles: np.ndarray, b: int, n: int) -> np.ndarray:
    n_tiles = tiles.shape[0]
    t32 = np.ascontiguousarray(tiles).view(np.uint32).reshape(n_tiles, b, 64, 4)
    streams = np.ascontiguousarray(t32.transpose(0, 2, 1, 3)).reshape(n_tiles, 64, 4 * b)
    tok = np.zeros((n_tiles, TILE, 128), np.int64)
    for L in range(64):
        for phi, p, dim in _v_lane_fields(L):
            field = _get(streams[:, L], 2 * b * phi, 2 * b)
            tok[:, p, dim] = field & ((1 << b) - 1)
            tok[:, p + 32, dim] = field >> b
    return tok.reshape(-1, 128)[:n]
