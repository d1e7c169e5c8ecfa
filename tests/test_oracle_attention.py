"""Pins for oracle.attention and oracle.pipeline (dequantization + fp64 decode)."""
import numpy as np
import pytest
from scipy.special import softmax

import synth
from oracle import attention, codebook, layout, pipeline


def _softmax_attention(q, K, V):
    """Independent reference: scipy's softmax over q.K^T/sqrt(d)."""
    return softmax(q @ K.T / np.sqrt(q.shape[-1]), axis=-1) @ V


def test_attend_matches_scipy_softmax():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((4, 128)) * 3
    K = rng.standard_normal((300, 128)); V = rng.standard_normal((300, 128))
    np.testing.assert_allclose(attention.attend(q, K, V), _softmax_attention(q, K, V), rtol=1e-12, atol=1e-13)


def test_invariants():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((2, 128)) * 2
    K = rng.standard_normal((50, 128)); V = rng.standard_normal((50, 128))
    o = attention.attend(q, K, V)
    perm = rng.permutation(50)
    np.testing.assert_allclose(attention.attend(q, K[perm], V[perm]), o, rtol=1e-12)  # A.V = A_P.V_P
    np.testing.assert_allclose(attention.attend(q, K[:1], V[:1]), np.repeat(V[:1], 2, 0), rtol=1e-15)
    np.testing.assert_allclose(attention.attend(np.zeros((1, 128)), K, V)[0], V.mean(0), rtol=1e-12)
    assert np.all(o <= V.max(0) + 1e-12) and np.all(o >= V.min(0) - 1e-12)


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 50])
def test_split_merge_equals_single_pass(splits):
    rng = np.random.default_rng(splits)
    q = rng.standard_normal((3, 128)) * 4
    K = rng.standard_normal((50, 128)); V = rng.standard_normal((50, 128))
    parts = [attention.partial(q, K[s], V[s]) for s in np.array_split(np.arange(50), splits)]
    np.testing.assert_allclose(attention.merge(parts), attention.attend(q, K, V), rtol=1e-12)


def test_dequant_closed_forms():
    b = 3
    c = codebook.codebook(b)[0].astype(np.float64)
    codes = np.tile(np.arange(8), 16)[None].repeat(2, 0)
    S = np.float16([1.5, 0.25])
    v = attention.dequant_codebook(codes, S, b)
    np.testing.assert_array_equal(v[0], 1.5 * c[codes[0]])
    bits = np.zeros(64, int); bits[3] = 3
    sigma = np.ones(64, np.float32) * np.float32(0.3)
    k = attention.dequant_k_gtq(codes, S, sigma, bits)
    assert np.count_nonzero(k[0]) == 2
    assert k[1, 6] == 0.25 * float(np.float32(0.3)) * c[codes[1, 6]]
    xa = attention.dequant_affine(np.array([[0, 3, 15] + [0] * 125]), np.float16([[0.5]]), np.float16([[-1.0]]), 128)
    np.testing.assert_array_equal(xa[0, :3], [-1.0, 0.5, 6.5])


def _layer(w, n, meta, n_recent=0):
    K = np.stack([synth.keys(w, 0, h, 0, n) for h in range(w.Hkv)])[None]
    V = np.stack([synth.values(w, 0, h, 0, n) for h in range(w.Hkv)])[None]
    q = np.concatenate([synth.queries(w, 0, h, 0, n) for h in range(w.Hkv)])[None]
    c = pipeline.build_layer(K, V, k_mode="gtq", v_mode="codebook", v_bits=w.v_bits, n_cap=n,
                             meta=meta, n_recent=n_recent)
    return K, V, q, c


def test_passthrough_width16_equals_unquantized_keys():
    """All blocks at the oracle-only width 16 (fp16 passthrough): the full pipeline (quantize ->
    pack -> unpack -> dequant -> attention) equals attention over fp16 keys and dequantized V."""
    w = synth.reduced(synth.WORKLOADS[1], N=200)
    meta = pipeline.LayerMeta(np.full((1, 64), 16), np.ones((1, 64), np.float32),
                              np.ones((1, 64), np.float32), np.ones((1, 64)))
    K, V, q, c = _layer(w, 200, meta)
    o = pipeline.decode_layer(c, q)
    vc, S = __import__("oracle").quantize.quantize_v(V[0, 0], w.v_bits)
    Vh = attention.dequant_codebook(vc, S, w.v_bits)
    ref = _softmax_attention(q[0].astype(np.float64), K[0, 0].astype(np.float16).astype(np.float64), Vh)
    np.testing.assert_allclose(o[0], ref, rtol=1e-12, atol=1e-12)


def test_recent_buffer_concatenation_position_free():
    w = synth.reduced(synth.WORKLOADS[5], N=300, L=1)
    kc = [synth.calibration(w, 0, h) for h in range(w.Hkv)]
    meta = pipeline.calibrate([a for a, _ in kc], [b for _, b in kc], w.k_budget_units)
    K, V, q, c = _layer(w, 300, meta, n_recent=64)
    assert c.n_packed == 236 and c.n_recent_valid == 64
    # ring slots: position p lives at slot p % 64
    np.testing.assert_array_equal(c.recent_k[0, 1, 299 % 64], K[0, 1, 299].astype(np.float16))
    o = pipeline.decode_layer(c, q)
    for h in range(w.Hkv):
        Kh, Vh = pipeline.dequant_head(c, 0, h)
        # recent tokens first instead of last: same result (A.V = A_P.V_P)
        Kr = np.concatenate([Kh[236:], Kh[:236]]); Vr = np.concatenate([Vh[236:], Vh[:236]])
        qh = q[0, h * w.g:(h + 1) * w.g].astype(np.float64)
        np.testing.assert_allclose(_softmax_attention(qh, Kr, Vr), o[0, h * w.g:(h + 1) * w.g], rtol=1e-10, atol=1e-12)
        # the recent part is the fp16 rows of positions 236..299, position p in ring slot p % 64
        for p in range(236, 300):
            np.testing.assert_array_equal(Kh[236 + p % 64], K[0, h, p].astype(np.float16).astype(np.float64))
            np.testing.assert_array_equal(Vh[236 + p % 64], V[0, h, p].astype(np.float16).astype(np.float64))


def test_block_gtq_beats_uniform_logit_mae():
    """Direction of the abstract's per-layer comparison: at equal K budget, per-block widths give a
    lower RoPE-logit MAE than uniform widths on heterogeneous synthetic heads (soft check)."""
    from oracle import quantize
    for wid in (1, 2):
        w = synth.reduced(synth.WORKLOADS[wid], N=2048)
        for h in range(w.Hkv):
            kc, qc = synth.calibration(w, 0, h)
            meta = pipeline.calibrate([kc], [qc], w.k_budget_units)
            K = synth.keys(w, 0, h, 0, 2048)
            q = synth.queries(w, 0, h, 0, 2048).astype(np.float64)
            exact = q @ K.astype(np.float64).T
            maes = []
            for bits in (meta.bits[0], np.full(64, w.k_budget_units // 64)):
                codes, S = quantize.quantize_k_gtq(K, meta.sigma[0], meta.r[0], bits)
                Kh = attention.dequant_k_gtq(codes, S, meta.sigma[0], bits)
                maes.append(np.abs(q @ Kh.T - exact).mean())
            assert maes[0] < maes[1], (wid, h, maes)


def test_affine_pipeline_matches_direct():
    from oracle import quantize
    w = synth.reduced(synth.WORKLOADS[4], N=130, Hkv=2, Hq=8)
    K = np.stack([synth.keys(w, 0, h, 0, 130) for h in range(2)])[None]
    V = np.stack([synth.values(w, 0, h, 0, 130) for h in range(2)])[None]
    q = np.concatenate([synth.queries(w, 0, h, 0, 130) for h in range(2)])[None]
    c = pipeline.build_layer(K, V, k_mode="affine", v_mode="affine", v_bits=2, n_cap=192, k_bits=4, k_group=32)
    o = pipeline.decode_layer(c, q)
    for h in range(2):
        kc, ks, kz = quantize.quantize_affine(K[0, h], 4, 32)
        vc, vs, vz = quantize.quantize_affine(V[0, h], 2, 128)
        ref = _softmax_attention(q[0, 4 * h:4 * h + 4].astype(np.float64),
                                 attention.dequant_affine(kc, ks, kz, 32), attention.dequant_affine(vc, vs, vz, 128))
        np.testing.assert_allclose(o[0, 4 * h:4 * h + 4], ref, rtol=1e-12, atol=1e-12)


# --- key rotation (affine keys) ---

def _signs(seed, d=128):
    return np.where(np.random.default_rng(seed).random(d) < 0.5, -1.0, 1.0)


def test_hadamard_matrix_and_fast_transform():
    """The fast transform's stages compute the Sylvester matrix: exact on integer inputs (no
    rounding), H H = 128 I, and the fp32 transform stays within its rounding bound."""
    from oracle import quantize
    H = attention.hadamard_matrix(128)
    np.testing.assert_array_equal(H @ H, 128 * np.eye(128))
    assert np.all(np.abs(H) == 1) and np.all(H[0] == 1) and np.all(H[:, 0] == 1)
    rng = np.random.default_rng(3)
    s = _signs(4)
    xi = rng.integers(-100, 100, (5, 128)).astype(np.float32)        # exact in fp32 throughout
    np.testing.assert_array_equal(quantize.hadamard_rotate_f32(xi, s), (xi * s) @ H.T / 16)
    x = rng.standard_normal((50, 128)).astype(np.float32)
    y = quantize.hadamard_rotate_f32(x, s).astype(np.float64)
    exact = (x.astype(np.float64) * s) @ H.T / 16
    bound = 7 * 2.0 ** -24 * (np.abs(x).astype(np.float64) @ np.abs(H).T) / 16
    assert np.all(np.abs(y - exact) <= bound)


def test_key_rotation_round_trip_and_logit_invariance():
    from oracle import quantize
    rng = np.random.default_rng(5)
    s = _signs(6)
    k = rng.standard_normal((20, 128))
    y = (k * s) @ attention.hadamard_matrix().T / 16                 # fp64 rotation
    np.testing.assert_allclose(attention.unrotate_keys(y, s), k, atol=1e-12)
    q = rng.standard_normal(128)
    qr = attention.hadamard_matrix() @ (q * s) / 8                   # the decode's query rotation
    np.testing.assert_allclose(y @ qr, k @ q, rtol=1e-12, atol=1e-12)
    yf = quantize.hadamard_rotate_f32(k.astype(np.float32), s)
    np.testing.assert_allclose(attention.unrotate_keys(yf, s), k.astype(np.float32), atol=1e-5)


def test_key_rotation_spreads_outlier_channels():
    """Soft check of the direction the summary reports: keys with a few large channels quantize
    with a lower error under 4-bit, group-32 affine groups once rotated (measured in the original
    key space after the exact inverse)."""
    from oracle import quantize
    rng = np.random.default_rng(11)
    k = rng.standard_normal((2000, 128)).astype(np.float32)
    k[:, [5, 77]] *= 20.0
    s = _signs(12)
    c0, s0, z0 = quantize.quantize_affine(k, 4, 32)
    e0 = np.mean((attention.dequant_affine(c0, s0, z0, 32) - k) ** 2)
    y = quantize.hadamard_rotate_f32(k, s)
    c1, s1, z1 = quantize.quantize_affine(y, 4, 32)
    e1 = np.mean((attention.unrotate_keys(attention.dequant_affine(c1, s1, z1, 32), s) - k) ** 2)
    assert e1 < 0.5 * e0


def test_rotated_affine_pipeline_matches_direct():
    """A rotated affine layer decodes to the same output as attention over its keys dequantized
    and rotated back by hand; ring tokens stay unrotated."""
    import synth
    from oracle import pipeline
    w = synth.reduced(synth.WORKLOADS[4], L=1, B=1, Hkv=2, Hq=8)
    N = 300
    K = np.stack([synth.keys(w, 0, h, 0, N) for h in range(2)])[None]
    V = np.stack([synth.values(w, 0, h, 0, N) for h in range(2)])[None]
    q = np.concatenate([synth.queries(w, 0, h, 0, N) for h in range(2)])[None]
    rot = np.stack([_signs(20 + h) for h in range(2)])
    oc = pipeline.build_layer(K, V, k_mode="affine", v_mode=w.v_mode, v_bits=w.v_bits, n_cap=320, k_bits=4,
                              k_group=32, n_recent=40, k_rot=rot)
    out = pipeline.decode_layer(oc, q)
    from oracle import layout, quantize
    for h in range(2):
        n = oc.n_packed
        codes = layout.k_affine_codes(layout.untile_records(oc.k_codes[0, h], n, 16), 4)
        Kr = attention.dequant_affine(codes, oc.k_scale[0, h, :n], oc.k_zero[0, h, :n], 32)
        y = quantize.hadamard_rotate_f32(K[0, h, :n], rot[h])
        c2, s2, z2 = quantize.quantize_affine(y, 4, 32)
        np.testing.assert_array_equal(codes, c2)
        Kx = np.concatenate([attention.unrotate_keys(Kr, rot[h]), oc.recent_k[0, h, :oc.n_recent_valid]])
        Vx = pipeline.dequant_head(oc, 0, h)[1]
        ref = attention.attend(q[0, 4 * h:4 * (h + 1)].astype(np.float64), Kx, Vx)
        np.testing.assert_allclose(out[0, 4 * h:4 * (h + 1)], ref, rtol=1e-12, atol=1e-12)


# --- value rotation ---

def test_hadamard_matrix_is_sylvester():
    """The oracle's Hadamard matrix is the Sylvester construction scipy builds."""
    from scipy.linalg import hadamard
    np.testing.assert_array_equal(attention.hadamard_matrix(128), hadamard(128))


def test_value_rotation_undone_once_on_the_output():
    """Values stored as y = H (s * v) / 16: attention over y, then s * (H o') / 8, equals attention
    over v (linearity); the signs go after the transform on the way back (before it, the output
    is wrong for random signs)."""
    rng = np.random.default_rng(21)
    s = _signs(22)
    H = attention.hadamard_matrix()
    q = rng.standard_normal((4, 128)) * 2
    K = rng.standard_normal((70, 128))
    V = rng.standard_normal((70, 128))
    Y = (V * s) @ H.T / 16                                            # fp64 rotation of every row
    o_rot = attention.attend(q, K, Y)
    np.testing.assert_allclose(attention.unrotate_output(o_rot, s), attention.attend(q, K, V), rtol=1e-12, atol=1e-12)
    wrong = (o_rot * s) @ H.T / 8
    assert np.max(np.abs(wrong - attention.attend(q, K, V))) > 1e-2
    np.testing.assert_allclose(attention.unrotate_output(Y, s), V, atol=1e-12)


@pytest.mark.parametrize("v_mode,v_bits", [("codebook", 3), ("affine", 2)])
def test_value_rotation_pipeline(v_mode, v_bits):
    """A layer with rotated values stores the codes of the rotated rows (fp32 fast transform) and
    decodes to attention over those values dequantized, rotated back once on the output."""
    from oracle import quantize
    w = synth.reduced(synth.WORKLOADS[2], L=1, v_mode=v_mode, v_bits=v_bits)
    N = 200
    m = pipeline.calibrate(*zip(*[synth.calibration(w, 0, h) for h in range(w.Hkv)]), w.k_budget_units)
    K = np.stack([synth.keys(w, 0, h, 0, N) for h in range(w.Hkv)])[None]
    V = np.stack([synth.values(w, 0, h, 0, N) for h in range(w.Hkv)])[None]
    q = np.concatenate([synth.queries(w, 0, h, 0, N) for h in range(w.Hkv)])[None]
    s = np.stack([_signs(30 + h) for h in range(w.Hkv)])
    c = pipeline.build_layer(K, V, k_mode="gtq", v_mode=v_mode, v_bits=v_bits, n_cap=256, meta=m, v_rot=s)
    for h in range(w.Hkv):
        y = quantize.hadamard_rotate_f32(V[0, h], s[h])
        if v_mode == "codebook":
            codes, S = quantize.quantize_v(y, v_bits)
            np.testing.assert_array_equal(c.v_scale[0, h, :N].view(np.uint16), S.view(np.uint16))
        else:
            codes, sc, zr = quantize.quantize_affine(y, v_bits, 128)
            np.testing.assert_array_equal(c.v_scale[0, h, :N].view(np.uint16), sc[:, 0].view(np.uint16))
        np.testing.assert_array_equal(layout.v_codes(c.v_codes[0, h], v_bits, N), codes)
    out = pipeline.decode_layer(c, q)
    for h in range(w.Hkv):
        Kh, Yh = pipeline.dequant_head(c, 0, h)
        g = w.Hq // w.Hkv
        ref = attention.unrotate_output(attention.attend(q[0, h * g:(h + 1) * g].astype(np.float64), Kh, Yh), s[h])
        np.testing.assert_allclose(out[0, h * g:(h + 1) * g], ref, rtol=1e-12, atol=1e-12)


def test_value_rotation_at_high_width_tracks_exact_attention():
    """8-bit codebook values under the rotation: the decode stays as close to attention over the
    unquantized values as the unrotated layer does (the rotation is undone, not left on the
    output, where the error would be of the output's own size)."""
    w = synth.reduced(synth.WORKLOADS[2], L=1, Hkv=1, Hq=8, v_bits=8)
    N = 150
    m = pipeline.calibrate(*zip(*[synth.calibration(w, 0, 0)]), w.k_budget_units)
    K = synth.keys(w, 0, 0, 0, N)[None, None]
    V = synth.values(w, 0, 0, 0, N)[None, None]
    q = synth.queries(w, 0, 0, 0, N)[None]
    err = {}
    for rot in (None, _signs(40)[None]):
        c = pipeline.build_layer(K, V, k_mode="gtq", v_mode="codebook", v_bits=8, n_cap=192, meta=m, v_rot=rot)
        Kh, _ = pipeline.dequant_head(c, 0, 0)
        exact = attention.attend(q[0].astype(np.float64), Kh, V[0, 0].astype(np.float64))
        err[rot is None] = np.max(np.abs(pipeline.decode_layer(c, q)[0] - exact))
    assert err[False] < 2 * err[True] and err[False] < 0.1 < np.abs(exact).max()


def test_value_rotation_refuses_the_fp16_window():
    K = np.zeros((1, 1, 10, 128), np.float32)
    with pytest.raises(ValueError):
        pipeline.build_layer(K, K, k_mode="affine", v_mode="affine", v_bits=2, n_cap=64, n_recent=4,
                             v_rot=np.ones((1, 128)))
