"""Pins for oracle.quantize (codes and scales) and oracle.layout (packed bytes)."""
import math

import numpy as np
import pytest

from oracle import codebook, layout, quantize

F32 = np.float32


def _row_whitened(x, r):
    return x.astype(np.float64) * np.repeat(r.astype(np.float64), 2)


@pytest.mark.parametrize("seed", range(4))
def test_k_codes_are_nearest_centroids(seed):
    rng = np.random.default_rng(seed)
    n = 500
    sigma = np.exp(rng.uniform(-3, 2, 64)).astype(F32)
    r = (F32(1) / sigma).astype(F32)
    bits = rng.integers(0, 9, 64)
    x = (rng.standard_normal((n, 128)) * np.repeat(sigma, 2)).astype(F32)
    codes, S = quantize.quantize_k_gtq(x, sigma, r, bits)
    # scale = fp16 RMS of the whitened row (within fp32 rounding of the sum, + fp16 half-ulp)
    rms = np.sqrt(np.mean(_row_whitened(x, r) ** 2, axis=1))
    S64 = S.astype(np.float64)
    assert np.all(np.abs(S64 - rms) <= 2.0 ** -11 * rms * 1.0001 + 1e-6 * rms)
    n_edge = 0
    for i in range(64):
        b = int(bits[i])
        if b == 0:
            assert np.all(codes[:, 2 * i:2 * i + 2] == 0)
            continue
        c16, thr = codebook.codebook(b)
        c = c16.astype(np.float64)
        for e in (0, 1):
            u = x[:, 2 * i + e].astype(np.float64) / (S64 * float(sigma[i]))
            nearest = np.argmin(np.abs(u[:, None] - c[None, :]), axis=1)
            bad = codes[:, 2 * i + e] != nearest
            if bad.any():  # only allowed within fp32 rounding of a decision threshold
                t = thr.astype(np.float64)
                dist = np.min(np.abs(u[bad, None] - t[None, :]), axis=1)
                assert np.all(dist <= 1e-6 * np.maximum(1, np.abs(u[bad]))), dist
                n_edge += int(bad.sum())
    assert n_edge < 5


def test_v_mse_matches_codebook():
    """Per-token normalised values: distortion / S^2 matches the table's N(0,1) MSE."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4000, 128)).astype(F32)
    for b in (1, 2, 3, 4):
        codes, S = quantize.quantize_v(x, b)
        c = codebook.codebook(b)[0].astype(np.float64)
        xh = S.astype(np.float64)[:, None] * c[codes]
        mse = np.mean(((x - xh) / S.astype(np.float64)[:, None]) ** 2)
        assert abs(mse - codebook.codebook_mse(b)) / codebook.codebook_mse(b) < 0.05


def test_scale_exact_on_exact_sums():
    """With integer inputs every partial sum is exact in fp32: S = fp16(sqrt(mean(x^2)))."""
    x = np.zeros((3, 128), F32)
    x[0, :] = 3.0
    x[1, ::2] = 2.0
    x[2, 5] = 64.0
    _, S = quantize.quantize_v(x, 2)
    want = [3.0, math.sqrt(2.0), math.sqrt(64.0 ** 2 / 128)]
    np.testing.assert_array_equal(S, np.float16(want))


def test_zero_row():
    x = np.zeros((2, 128), F32)
    codes, S = quantize.quantize_v(x, 3)
    assert np.all(S == 0)


def test_sequential_sum_order_matters():
    """The scale is a *sequential* fp32 sum: a row where pairwise and sequential sums differ."""
    x = np.zeros((1, 128), F32)
    x[0, 0] = 4096.0
    x[0, 1:] = 0.5
    _, S = quantize.quantize_v(x, 1)
    acc = F32(0)
    for v in x[0]:
        acc = F32(acc + F32(v * v))
    assert S[0] == np.float16(np.sqrt(F32(acc / F32(128))))


def test_affine_closed_forms():
    x = np.zeros((3, 128), F32)
    x[0] = np.linspace(-1, 2, 128, dtype=F32)
    x[1] = 0.75                                     # constant groups -> scale 0 -> code 0
    x[2] = np.random.default_rng(1).standard_normal(128).astype(F32)
    for b, G in ((4, 32), (2, 128), (8, 64)):
        codes, scale, zero = quantize.quantize_affine(x, b, G)
        assert codes.min() >= 0 and codes.max() <= 2 ** b - 1
        xg = x.reshape(3, -1, G)
        cg = codes.reshape(3, -1, G)
        # the group minimum maps to 0 and the maximum to the top code (row 0 and 2)
        for row in (0, 2):
            assert np.all(cg[row][np.arange(xg.shape[1]), xg[row].argmin(1)] == 0)
            assert np.all(cg[row][np.arange(xg.shape[1]), xg[row].argmax(1)] == 2 ** b - 1)
        assert np.all(scale[1] == 0) and np.all(codes[1] == 0)
        xh = np.repeat(scale.astype(np.float64), G, 1) * codes + np.repeat(zero.astype(np.float64), G, 1)
        err = np.abs(xh - x)
        lim = 0.5 * np.repeat(scale.astype(np.float64), G, 1) * (1 + 2 ** -9) + np.abs(
            np.repeat(zero.astype(np.float64), G, 1) - np.repeat(x.reshape(3, -1, G).min(-1), G, 1)) + 1e-7
        assert np.all(err[[0, 2]] <= lim[[0, 2]] + 2 ** -10 * (2 ** b) * np.repeat(scale.astype(np.float64), G, 1)[[0, 2]])


def test_affine_rounds_half_to_even():
    # group [0, 3] with b = 1: scale = 3, zero = 0; x = 1.5 -> 0.5 -> rint_even 0
    x = np.zeros((1, 128), F32)
    x[0, 1] = 3.0
    x[0, 2] = 1.5
    codes, scale, zero = quantize.quantize_affine(x, 1, 128)
    assert scale[0, 0] == 3.0 and codes[0, 2] == 0 and codes[0, 1] == 1


# ---------------------------------------------------------------- layout
def test_block_order_and_record_size():
    bits = np.zeros(64, int)
    bits[[5, 2, 9, 40]] = [3, 3, 8, 1]
    np.testing.assert_array_equal(layout.block_order(bits), [9, 2, 5, 40])
    assert layout.k_gtq_dwords(192) == 12 and layout.k_gtq_dwords(128) == 8


def test_k_record_hand_worked():
    """Widths: block 1 = 5 bits, block 0 = 3 bits, all others 0 except padding blocks to U=16.
    Block order: 1 (w5), 0 (w3), then 8 blocks of width 1 (blocks 2..9)."""
    bits = np.zeros(64, int)
    bits[0], bits[1] = 3, 5
    bits[2:10] = 1
    assert bits.sum() == 16
    codes = np.zeros((1, 128), int)
    codes[0, 2], codes[0, 3] = 0b10110, 0b00011   # block 1 -> bits [0,5) and [5,10)
    codes[0, 0], codes[0, 1] = 0b101, 0b011       # block 0 -> bits [10,13) and [13,16)
    codes[0, 4:20] = [1, 0] * 8                    # blocks 2..9: coordinate 2i = 1 at bits 16,18,...
    w = layout.k_gtq_words(codes, bits)
    want = 0b10110 | (0b00011 << 5) | (0b101 << 10) | (0b011 << 13) | sum(1 << (16 + 2 * k) for k in range(8))
    assert w.shape == (1, 1) and int(w[0, 0]) == want


@pytest.mark.parametrize("b", [2, 4, 8])
def test_affine_k_record_hand_worked(b):
    """Affine key record: coordinate j at bits [b*j, b*j + b) of a little-endian stream of b*4
    dwords, so dword k holds coordinates 32k/b .. 32(k+1)/b - 1, coordinate j at bit (b*j) % 32.
    Hand-built dwords: the codes 1, 2, 3, 0, ... (repeating mod 2^b) over the first dword, the top
    code 2^b - 1 in the last coordinate, zeros elsewhere except coordinate 32/b (the first of
    dword 1) set to 1."""
    per = 32 // b
    codes = np.zeros((1, 128), int)
    first = [(j + 1) % (1 << b) for j in range(per)]   # 1, 2, 3, 0 for b = 2; 1..8 for b = 4; 1..4 for b = 8
    codes[0, :per] = first
    codes[0, per] = 1
    codes[0, 127] = (1 << b) - 1
    w = layout.k_affine_words(codes, b)
    assert w.shape == (1, 4 * b)
    want0 = sum(v << (b * j) for j, v in enumerate(first))
    assert int(w[0, 0]) == want0
    assert int(w[0, 1]) == 1                            # coordinate 32/b at bit 0 of dword 1
    assert int(w[0, -1]) == ((1 << b) - 1) << (32 - b)  # coordinate 127 in the top bits
    assert not np.any(w[0, 2:-1])
    # spelled out per width
    if b == 2:
        assert int(w[0, 0]) == 0b00_11_10_01_00_11_10_01_00_11_10_01_00_11_10_01
    if b == 4:
        assert int(w[0, 0]) == 0x87654321
    if b == 8:
        assert int(w[0, 0]) == 0x04030201
    np.testing.assert_array_equal(layout.k_affine_codes(w, b), codes)


def test_straddling_field_round_trip():
    rng = np.random.default_rng(11)
    for _ in range(20):
        bits = np.zeros(64, int)
        while bits.sum() < 192:
            i = rng.integers(64)
            if bits[i] < 8:
                bits[i] += 1
        codes = np.zeros((70, 128), int)
        for i in range(64):
            if bits[i]:
                codes[:, 2 * i:2 * i + 2] = rng.integers(0, 2 ** bits[i], (70, 2))
        words = layout.k_gtq_words(codes, bits)
        assert words.shape == (70, 12)
        tiles = layout.tile_records(words, 2)
        back = layout.k_gtq_codes(layout.untile_records(tiles, 70, 12), bits)
        np.testing.assert_array_equal(back, codes)


def test_tile_record_positions():
    """Token t's dword k lives at byte (k*64 + t)*4 of its tile (dword-major, token-minor)."""
    for R in (12, 6, 8):
        words = np.arange(64 * R, dtype=np.uint32).reshape(64, R) * 7 + 1
        tiles = layout.tile_records(words, 1).view(np.uint32)[0]
        for t in (0, 1, 37, 63):
            for k in range(R):
                assert tiles[k * 64 + t] == words[t, k]
    words = np.arange(100 * 8, dtype=np.uint32).reshape(100, 8)
    tiles = layout.tile_records(words, 2)
    np.testing.assert_array_equal(layout.untile_records(tiles, 100, 8), words)
    assert tiles.view(np.uint32)[1, 3 * 64 + (70 - 64)] == words[70, 3]


def test_v_lane_stream_layout_hand_worked():
    """Positions worked out by hand from the layout rule (b = 3, 2b = 6-bit fields)."""
    b = 3
    codes = np.zeros((60, 128), int)
    # token 5 = pair p 5 (s 0, j 1, m 1), low half; dim 17 = (db 1, dd 1): lane 17, field 5 at
    # bit 30 -> straddles stream dwords 0 and 1 -> tile dwords 68 and 69
    codes[5, 17] = 5
    # token 40 = p 8 + 32 (s 0, j 2, m 0), high half; dim 127 = (db 7, dd 15): lane 47, field 28
    # at bit 168 -> stream dword 5 bit 8 -> tile dword (64 + 47)*4 + 1 = 445
    codes[40, 127] = 6
    # tokens 20 and 52 = p 20 (s 1, j 1, m 0), both halves; dim 0: lane 16, field 32 at bit 192
    # -> stream dword 6 bit 0 -> tile dword (64 + 16)*4 + 2 = 322
    codes[20, 0], codes[52, 0] = 7, 3
    tiles = layout.v_tiles(codes, b, 1).view(np.uint32)[0]
    assert tiles[68] == 1 << 30 and tiles[69] == 1
    assert tiles[445] == 48 << 8
    assert tiles[322] == 7 | (3 << 3)
    assert np.count_nonzero(tiles) == 4
    np.testing.assert_array_equal(layout.v_codes(layout.v_tiles(codes, b, 1), b, 60), codes)


def test_v_lane_fields_cover_tile_once():
    """Every (token, dim) of a tile appears in exactly one field of exactly one lane stream."""
    seen = np.zeros((64, 128), int)
    for L in range(64):
        phis = [phi for phi, _, _ in layout._v_lane_fields(L)]
        assert sorted(phis) == list(range(64))
        for _, p, dim in layout._v_lane_fields(L):
            seen[p, dim] += 1
            seen[p + 32, dim] += 1
    assert (seen == 1).all()


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_v_round_trip(b):
    rng = np.random.default_rng(b)
    codes = rng.integers(0, 2 ** b, (129, 128))
    np.testing.assert_array_equal(layout.v_codes(layout.v_tiles(codes, b, 3), b, 129), codes)


def test_bytes_per_token():
    """K3V3 = 48+2+48+2; K2V2 = 68; affine K4 g32 + V2 g128 = 64+8+8+32+2+2; K4V2 is 75% of
    K4V4 in code bytes (the "Quantize What Counts" summary: 25% less KV memory)."""
    per_tok = lambda kb, vb: 4 * layout.k_gtq_dwords(kb * 64) + 2 + 16 * vb + 2
    assert per_tok(3, 3) == 100 and per_tok(2, 2) == 68
    assert 128 * 4 // 8 + 4 * 2 * 2 + 128 * 2 // 8 + 2 * 2 == 116
    k4, v2, v4 = 128 * 4 // 8, 128 * 2 // 8, 128 * 4 // 8
    assert (k4 + v2) / (k4 + v4) == 0.75
