"""Host-side checks of the C ABI that need no GPU: exports, tables, allocator, sizes, validation."""
import ctypes as C
import math
import re
import os

import numpy as np
import pytest

import packed_cache_decode_block_amd as P
from packed_cache_decode_block_amd import _lib
from oracle import allocate as oalloc
from oracle import codebook as ocb

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "bgtq.h")


def test_exports_every_declared_symbol():
    decl = set(re.findall(r"\b(bgtq_[a-z0-9_]+)\s*\(", open(HEADER).read()))
    assert decl == set(P.SYMBOLS)
    for name in decl:
        assert hasattr(P.lib, name)
    assert P.bgtq_version().startswith("bgtq")


@pytest.mark.parametrize("b", range(1, 9))
def test_codebook_tables_match_oracle(b):
    c16, thr = P.bgtq_codebook(b)
    oc, ot = ocb.codebook(b)
    np.testing.assert_array_equal(c16.view(np.uint16), oc.view(np.uint16))
    np.testing.assert_array_equal(thr.view(np.uint32), ot.view(np.uint32))


def _golden_rows():
    rows = {}
    for line in open(os.path.join(os.path.dirname(__file__), "golden", "lloyd_max_gaussian.txt")):
        if line.startswith("#") or not line.strip():
            continue
        b, cents, thr, _ = [f.strip() for f in line.split("|")]
        rows[int(b)] = ([float(x) for x in cents.split()], [float(x) for x in thr.split()])
    return rows


def _fp16_ulp(x):
    return float(np.spacing(np.float16(abs(x))))


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_library_codebook_matches_textbook(b):
    """The library's own table against Max (1960), Table I: each printed centroid and threshold
    within half a unit of its 4th digit plus half an fp16 ulp (the table is fp16-rounded)."""
    cents, thr = _golden_rows()[b]
    c16, t32 = P.bgtq_codebook(b)
    c = c16.astype(np.float64)
    h = len(c) // 2
    np.testing.assert_array_equal(c[:h], -c[::-1][:h])  # symmetric
    for got, want in zip(c[h:], cents):
        assert abs(got - want) <= 0.5 * 10 ** (math.floor(math.log10(want)) - 3) + 0.5 * _fp16_ulp(want), (got, want)
    for got, want in zip(t32.astype(np.float64)[h:], thr):
        assert abs(got - want) <= 0.5 * 10 ** (math.floor(math.log10(want)) - 3) + 0.5 * _fp16_ulp(want), (got, want)


@pytest.mark.parametrize("b", range(1, 9))
def test_library_codebook_centroid_condition(b):
    """Every library centroid is the mean of N(0,1) over its own cell (cell ends = the library's
    thresholds), up to the fp16 rounding of the centroids: within 1.5 fp16 ulps.  Thresholds are
    the exact midpoints of adjacent centroids.  Cell means by adaptive quadrature."""
    from scipy import integrate
    c16, t32 = P.bgtq_codebook(b)
    c = c16.astype(np.float64)
    t = t32.astype(np.float64)
    np.testing.assert_array_equal(t, 0.5 * (c[:-1] + c[1:]))
    assert np.all(np.diff(c) > 0)
    edges = np.concatenate([[-np.inf], t, [np.inf]])
    pdf = lambda x: math.exp(-0.5 * x * x) / math.sqrt(2 * math.pi)
    for m in range(len(c) // 2, len(c)):
        lo, hi = edges[m], edges[m + 1]
        mass = integrate.quad(pdf, lo, hi, epsabs=0, epsrel=1e-12)[0]
        first = integrate.quad(lambda x: x * pdf(x), lo, hi, epsabs=0, epsrel=1e-12)[0]
        assert abs(first / mass - c[m]) <= 1.5 * _fp16_ulp(c[m]), (m, first / mass, c[m])


def test_codebook_rejects_bad_width():
    with pytest.raises(P.BgtqError) as e:
        P.bgtq_codebook(9)
    assert e.value.code == P.E_INVALID


@pytest.mark.parametrize("seed", range(30))
def test_allocate_bit_exact_vs_oracle(seed):
    rng = np.random.default_rng(seed)
    n_heads = int(rng.integers(1, 5))
    s = np.exp(rng.uniform(-12, 12, (n_heads, 64)))
    if seed % 3 == 0:
        s[:, rng.integers(0, 64, 10)] = 0.0                      # dead blocks
    if seed % 4 == 0:
        s = np.round(s, 0) + 1.0                                 # ties
    U = int(rng.choice([64, 128, 192, 256]))
    got = P.bgtq_allocate(s, U)
    for h in range(n_heads):
        np.testing.assert_array_equal(got[h], oalloc.greedy(s[h], U, 8).astype(np.uint8))


def _lloyd_rate():
    return [1.0] + [ocb.codebook_mse(b) for b in range(1, 9)]


@pytest.mark.parametrize("seed", range(20))
def test_allocate_rate_bit_exact_vs_oracle(seed):
    rng = np.random.default_rng(700 + seed)
    n_heads = int(rng.integers(1, 4))
    s = np.exp(rng.uniform(-12, 12, (n_heads, 64)))
    if seed % 3 == 0:
        s[:, rng.integers(0, 64, 10)] = 0.0                      # dead blocks
    if seed % 4 == 0:
        s = np.round(s, 0) + 1.0                                 # ties
    U = int(rng.choice([64, 128, 192, 256]))
    b_min = 1 if seed % 5 == 0 else 0
    rate = _lloyd_rate()
    got = P.bgtq_allocate(s, U, b_min=b_min, rate=rate)
    for h in range(n_heads):
        np.testing.assert_array_equal(got[h], oalloc.greedy_rate(s[h], U, rate, 8, b_min).astype(np.uint8))


def test_allocate_rate_errors():
    s = np.array([[1.0, 2.0, 3.0]])
    for bad in ([1.0, 0.5, 0.4, 0.1], [1.0, 0.5, 0.5, 0.4], [1.0, 0.5, np.nan, 0.1]):
        with pytest.raises(P.BgtqError) as e:
            P.bgtq_allocate(s, 3, b_max=3, rate=bad)
        assert e.value.code == P.E_INVALID
    with pytest.raises(P.BgtqError) as e:
        P.bgtq_allocate(s, 10, b_max=3, rate=[1.0, 0.4, 0.1, 0.05])   # 3 blocks x 3 bits < 10
    assert e.value.code == P.E_BUDGET
    rc = P.lib.bgtq_allocate_rate(s.ctypes.data_as(C.POINTER(C.c_double)), 1, 3, 3, 0, 3, None,
                                  np.zeros(3, np.uint8).ctypes.data_as(C.POINTER(C.c_uint8)))
    assert rc == P.E_INVALID


def test_allocate_b_min_and_errors():
    s = np.array([[1.0, 2.0, 0.0, 4.0]])
    got = P.bgtq_allocate(s, 9, b_min=2, b_max=4)
    np.testing.assert_array_equal(got[0], oalloc.greedy(s[0], 9, 4, b_min=2))
    with pytest.raises(P.BgtqError) as e:
        P.bgtq_allocate(s, 13, b_max=4)                          # 3 live blocks x 4 bits = 12 < 13
    assert e.value.code == P.E_BUDGET
    with pytest.raises(P.BgtqError) as e:
        P.bgtq_allocate(np.array([[1.0, -1.0]]), 2)
    assert e.value.code == P.E_INVALID
    with pytest.raises(P.BgtqError) as e:
        P.bgtq_allocate(np.array([[1.0, np.nan]]), 2)
    assert e.value.code == P.E_INVALID
    with pytest.raises(P.BgtqError):
        P.bgtq_allocate(s, 4, b_max=9)


def _desc(**kw):
    d = _lib.CacheDesc()
    base = dict(L=2, B=3, Hq=16, Hkv=2, d=128, n_cap=4096, k_mode=0, budget_units=192, k_bits=4, k_group=32,
                v_mode=0, v_bits=3, n_recent=0)
    base.update(kw)
    for k, v in base.items():
        setattr(d, k, v)
    return d


def test_cache_bytes_geometry():
    d = _desc()
    nb = lambda w: P.lib.bgtq_cache_bytes(C.byref(d), w)
    assert nb(_lib.BUF_K_CODES) == 2 * 3 * 2 * 4096 * 48          # 48 B per token (K3)
    assert nb(_lib.BUF_V_CODES) == 2 * 3 * 2 * 4096 * 48          # 3 bits x 128
    assert nb(_lib.BUF_K_SCALE) == 2 * 3 * 2 * 4096 * 2
    assert nb(_lib.BUF_K_ZERO) == 0
    d = _desc(k_mode=1, k_bits=4, k_group=32, v_mode=1, v_bits=2, n_recent=256)
    assert nb(_lib.BUF_K_CODES) == 2 * 3 * 2 * 4096 * 64
    assert nb(_lib.BUF_K_SCALE) == 2 * 3 * 2 * 4096 * 4 * 2
    assert nb(_lib.BUF_K_ZERO) == nb(_lib.BUF_K_SCALE)
    assert nb(_lib.BUF_V_ZERO) == 2 * 3 * 2 * 4096 * 2
    assert nb(_lib.BUF_RECENT_K) == 2 * 3 * 2 * 256 * 128 * 2


@pytest.mark.parametrize("kw,code", [
    (dict(d=64), P.E_UNSUPPORTED), (dict(Hq=15), P.E_INVALID), (dict(Hq=32, Hkv=2), P.E_UNSUPPORTED),
    (dict(n_cap=100), P.E_INVALID), (dict(budget_units=100), P.E_INVALID), (dict(v_bits=5), P.E_INVALID),
    (dict(k_mode=1, k_bits=3), P.E_INVALID), (dict(k_mode=1, k_group=48), P.E_INVALID), (dict(B=65), P.E_UNSUPPORTED),
    (dict(k_mode=7), P.E_INVALID), (dict(n_recent=-1), P.E_INVALID),
    (dict(k_rot=0x1000), P.E_UNSUPPORTED)])                        # key rotation needs affine keys
def test_descriptor_validation(kw, code):
    d = _desc(**kw)
    assert P.lib.bgtq_cache_bytes(C.byref(d), _lib.BUF_K_CODES) == code
    assert P.lib.bgtq_last_error()


def test_key_rotation_accepted_with_affine_keys():
    d = _desc(k_mode=1, k_bits=4, k_group=32, k_rot=0x1000)
    assert P.lib.bgtq_cache_bytes(C.byref(d), _lib.BUF_K_CODES) == 2 * 3 * 2 * 4096 * 64


def test_append_and_decode_validate_before_launch():
    """Invalid calls return an error without touching the device (NULL device pointers are never used)."""
    d = _desc()
    nt = np.zeros((2, 3), np.int64)
    d.n_tokens = nt.ctypes.data_as(C.POINTER(C.c_int64))
    fake = C.c_void_p(0x1000)
    # NULL cache buffers; then everything but the inverse key scales
    assert P.lib.bgtq_quantize_append(C.byref(d), 0, fake, fake, 2, 10, None, None) == P.E_INVALID
    for name in ("k_codes", "v_codes", "k_scale", "v_scale", "bits", "sigma"):
        setattr(d, name, 0x1000)
    assert P.lib.bgtq_quantize_append(C.byref(d), 0, fake, fake, 2, 10, None, None) == P.E_INVALID
    assert b"inv_sigma" in P.lib.bgtq_last_error()
    for name in ("k_codes", "v_codes", "k_scale", "v_scale", "bits", "sigma", "inv_sigma", "plan"):
        setattr(d, name, 0x1000)
    assert P.lib.bgtq_quantize_append(C.byref(d), 5, fake, fake, 2, 10, None, None) == P.E_INVALID  # layer
    assert P.lib.bgtq_quantize_append(C.byref(d), 0, fake, fake, 9, 10, None, None) == P.E_INVALID  # dtype
    assert P.lib.bgtq_quantize_append(C.byref(d), 0, fake, fake, 2, 5000, None, None) == P.E_CAPACITY
    assert (nt == 0).all()                                        # no side effect on failure
    out = C.c_void_p(0x2000)
    ws = C.c_void_p(0x10000)
    # empty context
    assert P.lib.bgtq_decode_attention(C.byref(d), 0, fake, 2, out, ws, 1 << 30, 4, None) == P.E_INVALID
    nt[0] = 100
    # misaligned / too small workspace
    assert P.lib.bgtq_decode_attention(C.byref(d), 0, fake, 2, out, C.c_void_p(0x10010), 1 << 30, 4, None) == P.E_INVALID
    assert P.lib.bgtq_decode_attention(C.byref(d), 0, fake, 2, out, ws, 16, 4, None) == P.E_INVALID
    # unsupported decode format (budget 208 -> 13-dword records has no kernel)
    d2 = _desc(budget_units=208)
    for name in ("k_codes", "v_codes", "k_scale", "v_scale", "bits", "sigma", "inv_sigma", "plan"):
        setattr(d2, name, 0x1000)
    d2.n_tokens = nt.ctypes.data_as(C.POINTER(C.c_int64))
    assert P.lib.bgtq_decode_attention(C.byref(d2), 0, fake, 2, out, ws, 1 << 30, 4, None) == P.E_UNSUPPORTED


def test_energy_and_fp16_validation():
    fake = C.c_void_p(0x1000)
    nul = None
    assert P.lib.bgtq_block_energy(nul, fake, 2, 10, 2, 8, 128, 0, None, None, None, fake, 4096, None) == P.E_INVALID
    assert P.lib.bgtq_block_energy(fake, fake, 2, 10, 2, 8, 64, 0, None, None, None, fake, 4096, None) == P.E_UNSUPPORTED
    assert P.lib.bgtq_block_energy(fake, fake, 2, 10, 2, 8, 128, 0, None, None, None, fake, 16, None) == P.E_INVALID
    assert P.lib.bgtq_fp16_decode_attention(fake, fake, 100, 1, 16, 2, 128, fake, 2, fake, C.c_void_p(0x10000), 16, 4,
                                            None) == P.E_INVALID
    assert P.lib.bgtq_fp16_decode_attention(fake, fake, 100, 1, 48, 2, 128, fake, 2, fake, C.c_void_p(0x10000),
                                            1 << 30, 4, None) == P.E_UNSUPPORTED
