"""GPU parity: HIP library vs the CPU oracle on the same seeded inputs (through the C ABI).

Bit-exact: packed code bytes and fp16 scales (and the fp16 ring).  Outputs: |gpu - ref| <=
2e-3 + 1e-3*|ref| elementwise, ref = float64 oracle attention over the oracle's own cache.
"""
import numpy as np
import pytest

import synth
from oracle import pipeline
from tests import _parity as T

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import packed_cache_decode_block_amd as P  # noqa: E402


def _compare_cache(cache, oc, w, layer=0, L=1):
    B, H = w.B, w.Hkv
    kc = T.layer_view(cache.k_codes, L, layer, oc.k_codes.shape).cpu().numpy()
    vc = T.layer_view(cache.v_codes, L, layer, oc.v_codes.shape).cpu().numpy()
    ks = T.layer_view(cache.k_scale, L, layer, oc.k_scale.shape).cpu().numpy()
    vs = T.layer_view(cache.v_scale, L, layer, oc.v_scale.shape).cpu().numpy()
    np.testing.assert_array_equal(ks.view(np.uint16), oc.k_scale.view(np.uint16), "k scales")
    np.testing.assert_array_equal(vs.view(np.uint16), oc.v_scale.view(np.uint16), "v scales")
    np.testing.assert_array_equal(kc, oc.k_codes, "k codes")
    np.testing.assert_array_equal(vc, oc.v_codes, "v codes")
    if oc.k_zero is not None:
        kz = T.layer_view(cache.k_zero, L, layer, oc.k_zero.shape).cpu().numpy()
        np.testing.assert_array_equal(kz.view(np.uint16), oc.k_zero.view(np.uint16), "k zeros")
    if oc.v_zero is not None:
        vz = T.layer_view(cache.v_zero, L, layer, oc.v_zero.shape).cpu().numpy()
        np.testing.assert_array_equal(vz.view(np.uint16), oc.v_zero.view(np.uint16), "v zeros")
    if oc.recent_k is not None:
        rk = T.layer_view(cache.recent_k, L, layer, oc.recent_k.shape).cpu().numpy()
        rv = T.layer_view(cache.recent_v, L, layer, oc.recent_v.shape).cpu().numpy()
        np.testing.assert_array_equal(rk.view(np.uint16), oc.recent_k.view(np.uint16), "recent k")
        np.testing.assert_array_equal(rv.view(np.uint16), oc.recent_v.view(np.uint16), "recent v")


CASES = {
    # name: (workload id, overrides, N, chunks)
    "w1_full": (1, {}, 4096, (None,)),
    "w1_ragged_chunks": (1, {}, 1000, (1, 2, 61, 64, 129, None)),
    "w2_reduced": (2, {"L": 1}, 4096 + 37, (None,)),
    "w3_reduced": (3, {"L": 1, "B": 2}, 2048 + 5, (777, None)),
    "w4_reduced": (4, {"L": 1, "B": 2}, 2048 + 13, (None,)),
    "w5_reduced": (5, {}, 3000, (1000, 7, None)),
    "w5_all_recent": (5, {}, 200, (None,)),
    # fp16 windows: the merge attends to windows of up to 512 rows itself (two token blocks per
    # wave at 512; one query head per kv head on the vector path; 4 per kv head with a ragged
    # window), a longer window takes a split-K launch of its own
    "w5_window_512": (5, {"n_recent": 512}, 1500 + 11, (600, None)),
    "w1_window_g1": (1, {"n_recent": 100}, 1000 + 1, (None,)),
    "w3_window_77": (3, {"L": 1, "B": 2, "n_recent": 77}, 500 + 3, (300, None)),
    "w5_window_600": (5, {"n_recent": 600}, 2000 + 5, (700, None)),
    # other matrix-core template shapes: 16-dword key records with 4-bit values (one value buffer),
    # and 4 query heads per kv head with 12-dword records and 3-bit values
    "w2_k4v4": (2, {"L": 1, "v_bits": 4, "k_budget_units": 256}, 1500 + 3, (None,)),
    "w3_k3v3": (3, {"L": 1, "B": 1, "v_bits": 3, "k_budget_units": 192}, 1000 + 9, (700, None)),
    # affine keys on the matrix cores: groups of 32 at 8 query heads per kv head with affine and with
    # codebook values; groups of 64 and 128 (k-steps accumulate within a group); groups of 64 at 2
    # query heads per kv head (the vector kernel)
    "w4_g8": (4, {"L": 1, "B": 1, "Hq": 16, "Hkv": 2}, 777, (None,)),
    "w4_g8_codebook_v3": (4, {"L": 1, "B": 1, "Hq": 16, "Hkv": 2, "v_mode": "codebook", "v_bits": 3}, 1000 + 3, (None,)),
    "w4_group64": (4, {"L": 1, "B": 1, "k_group": 64}, 600 + 1, (None,)),
    "w4_group128_g8": (4, {"L": 1, "B": 1, "k_group": 128, "Hq": 16, "Hkv": 2}, 500 + 7, (None,)),
    "w4_group64_g2_vector": (4, {"L": 1, "B": 1, "k_group": 64, "Hq": 4, "Hkv": 2}, 300 + 9, (None,)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_quantize_and_decode(name):
    wid, ov, N, chunks = CASES[name]
    w = synth.reduced(synth.WORKLOADS[wid], **ov)
    print(f"[case {name}] N={N} B={w.B} Hq={w.Hq} Hkv={w.Hkv}", flush=True)
    n_cap = ((N + 63) // 64 + 1) * 64
    m = T.meta(w, 0)
    K, V, q = T.inputs(w, 0, N)
    oc = T.oracle_layer(w, K, V, m, n_cap)
    cache = T.gpu_cache(w, n_cap)
    if m is not None:
        cache.set_metadata(0, m.bits, m.sigma, m.r)
    T.append_all(cache, 0, K, V, w.dtype, chunks)
    _compare_cache(cache, oc, w)
    ref = pipeline.decode_layer(oc, q)
    qd = T.to_dev(q, w.dtype)
    for ns in (0, 1, 3):
        out = cache.decode_attention(0, qd, n_splits=ns)
        torch.cuda.synchronize()
        e = T.assert_close(out.cpu().numpy(), ref, f"{name} splits={ns}")
        print(f"  splits={ns}: max abs err {e:.2e}", flush=True)


VECTOR_CASES = ["w2_reduced", "w3_k3v3", "w2_k4v4", "w4_g8", "w5_reduced"]


@pytest.mark.parametrize("name", VECTOR_CASES)
def test_vector_decode_path(name):
    """The cache's vector-ALU decode path (no matrix-core instructions) against the oracle, at the
    head ratios where the library otherwise takes the matrix cores; the matrix-core result of the
    same cache is compared too."""
    wid, ov, N, chunks = CASES[name]
    w = synth.reduced(synth.WORKLOADS[wid], **ov)
    print(f"[vector {name}] N={N} B={w.B} Hq={w.Hq} Hkv={w.Hkv}", flush=True)
    n_cap = ((N + 63) // 64 + 1) * 64
    m = T.meta(w, 0)
    K, V, q = T.inputs(w, 0, N)
    oc = T.oracle_layer(w, K, V, m, n_cap)
    cache = T.gpu_cache(w, n_cap)
    if m is not None:
        cache.set_metadata(0, m.bits, m.sigma, m.r)
    T.append_all(cache, 0, K, V, w.dtype, chunks)
    ref = pipeline.decode_layer(oc, q)
    qd = T.to_dev(q, w.dtype)
    auto = cache.decode_attention(0, qd).cpu().numpy()
    cache.decode_path = P.DECODE_VECTOR
    for ns in (0, 1, 3):
        out = cache.decode_attention(0, qd, n_splits=ns)
        torch.cuda.synchronize()
        e = T.assert_close(out.cpu().numpy(), ref, f"vector {name} splits={ns}")
        print(f"  splits={ns}: max abs err {e:.2e}", flush=True)
    T.assert_close(auto, ref, f"auto {name}")


def _widths(spec, seed):
    """Fixed allocation: spec = [(width, count), ...] over the 64 blocks (the rest get 0), placed in
    a seeded block order so that the stream order is not the block order."""
    bits = np.zeros(64, np.int64)
    order = np.random.default_rng(seed).permutation(64)
    i = 0
    for wd, cnt in spec:
        bits[order[i:i + cnt]] = wd
        i += cnt
    return bits


FIXED_CASES = {
    # name: (workload id, overrides, width spec, N).  The calibrated allocations of the workloads
    # leave 37..50 nonzero slots, so these shapes exercise what they do not: all 64 slots (four
    # k-steps), records without coordinate columns, records of coordinate columns only, a single
    # k-step, and the pair/coordinate boundary between widths 5 and 6 inside one k-step.
    "uniform_k3_g8": (2, {"L": 1}, [(3, 64)], 1500 + 7),
    "uniform_k2_g4": (3, {"L": 1, "B": 1, "v_bits": 2, "k_budget_units": 128}, [(2, 64)], 1000 + 3),
    "uniform_k4_v4_g8": (2, {"L": 1, "v_bits": 4, "k_budget_units": 256}, [(4, 64)], 700 + 11),
    "wide_only_g8": (2, {"L": 1}, [(8, 24)], 900 + 1),
    "one_kstep_g4": (3, {"L": 1, "B": 1, "v_bits": 2, "k_budget_units": 128}, [(8, 16)], 500 + 5),
    "widths_5_6_g8": (2, {"L": 1}, [(6, 16), (5, 16), (2, 8)], 1200 + 9),
    "widths_1_to_8_g8": (2, {"L": 1}, [(8, 4), (7, 4), (6, 4), (5, 4), (4, 4), (3, 16), (2, 8), (1, 8)], 800 + 2),
}


@pytest.mark.parametrize("name", list(FIXED_CASES))
def test_fixed_allocation_decode(name):
    """Uniform (TQ-MSE-style, every block at the same width) and hand-made Block-GTQ allocations
    through the same quantize and decode kernels, against the oracle."""
    wid, ov, spec, N = FIXED_CASES[name]
    w = synth.reduced(synth.WORKLOADS[wid], **ov)
    bits = np.stack([_widths(spec, 17 + h) for h in range(w.Hkv)])
    assert np.all(bits.sum(axis=1) == w.k_budget_units)
    print(f"[fixed {name}] N={N} Hq={w.Hq} Hkv={w.Hkv} nonzero={(bits[0] > 0).sum()}", flush=True)
    cal = T.meta(w, 0)
    m = pipeline.LayerMeta(bits, cal.sigma, cal.r, cal.scores)
    n_cap = ((N + 63) // 64) * 64
    K, V, q = T.inputs(w, 0, N)
    oc = T.oracle_layer(w, K, V, m, n_cap)
    cache = T.gpu_cache(w, n_cap)
    cache.set_metadata(0, m.bits, m.sigma, m.r)
    T.append_all(cache, 0, K, V, w.dtype)
    _compare_cache(cache, oc, w)
    ref = pipeline.decode_layer(oc, q)
    qd = T.to_dev(q, w.dtype)
    for ns in (0, 1, 3):
        out = cache.decode_attention(0, qd, n_splits=ns)
        torch.cuda.synchronize()
        e = T.assert_close(out.cpu().numpy(), ref, f"{name} splits={ns}")
        print(f"  splits={ns}: max abs err {e:.2e}", flush=True)


ROT_CASES = {
    # affine K4 keys stored rotated (QWC summary, Results: key-only rotation at K4V2); with and
    # without the fp16 recent ring (ring rows are evicted through the rotated quantizer, the ring
    # split itself attends with the unrotated query)
    "w4_rotated": (4, {"L": 1, "B": 2}, 2048 + 13, (None,)),
    "w4_rotated_ring": (4, {"L": 1, "B": 1, "n_recent": 64}, 1000 + 7, (300, 1, 64, None)),
}


@pytest.mark.parametrize("name", list(ROT_CASES))
def test_rotated_affine_keys(name):
    wid, ov, N, chunks = ROT_CASES[name]
    w = synth.reduced(synth.WORKLOADS[wid], **ov)
    print(f"[rotated {name}] N={N} B={w.B} Hq={w.Hq} Hkv={w.Hkv} n_recent={w.n_recent}", flush=True)
    n_cap = ((N + 63) // 64 + 1) * 64
    signs = np.where(np.random.default_rng(31).random((w.Hkv, 128)) < 0.5, -1.0, 1.0)
    K, V, q = T.inputs(w, 0, N)
    oc = pipeline.build_layer(K, V, k_mode=w.k_mode, v_mode=w.v_mode, v_bits=w.v_bits, n_cap=n_cap, k_bits=w.k_bits,
                              k_group=w.k_group, n_recent=w.n_recent, k_rot=signs)
    cache = P.PackedCache(L=1, B=w.B, Hq=w.Hq, Hkv=w.Hkv, n_cap=n_cap, k_mode=P.K_AFFINE, k_bits=w.k_bits,
                          k_group=w.k_group, v_mode=P.V_CODEBOOK if w.v_mode == "codebook" else P.V_AFFINE,
                          v_bits=w.v_bits, n_recent=w.n_recent, k_rotation=True)
    cache.set_key_rotation(0, signs)
    T.append_all(cache, 0, K, V, w.dtype, chunks)
    _compare_cache(cache, oc, w)
    ref = pipeline.decode_layer(oc, q)
    qd = T.to_dev(q, w.dtype)
    for ns in (0, 1, 3):
        out = cache.decode_attention(0, qd, n_splits=ns)
        torch.cuda.synchronize()
        e = T.assert_close(out.cpu().numpy(), ref, f"{name} splits={ns}")
        print(f"  splits={ns}: max abs err {e:.2e}", flush=True)


VROT_CASES = {
    # values stored rotated (QWC summary, Results: rotation integration; the summary finds the
    # value-only rotation marginal, built for comparison): codebook values with Block-GTQ keys at 8
    # and 4 query heads per kv head (the latter with two sequences and chunked appends, including
    # few-token ones that take the bulk quantizer), affine values with rotated affine keys
    "gtq_v3_g8": (2, {"L": 1}, 1500 + 7, (None,), False),
    "gtq_v2_g4_b2": (3, {"L": 1, "B": 2}, 700 + 3, (1, 5, 300, None), False),
    "affine_k4v2_both_rotated": (4, {"L": 1, "B": 1}, 900 + 1, (None,), True),
}


@pytest.mark.parametrize("name", list(VROT_CASES))
def test_rotated_values(name):
    wid, ov, N, chunks, krot = VROT_CASES[name]
    w = synth.reduced(synth.WORKLOADS[wid], **ov)
    print(f"[rotated values {name}] N={N} B={w.B} Hq={w.Hq} Hkv={w.Hkv} keys rotated {krot}", flush=True)
    n_cap = ((N + 63) // 64 + 1) * 64
    vs = np.where(np.random.default_rng(41).random((w.Hkv, 128)) < 0.5, -1.0, 1.0)
    ks = np.where(np.random.default_rng(43).random((w.Hkv, 128)) < 0.5, -1.0, 1.0) if krot else None
    m = T.meta(w, 0)
    K, V, q = T.inputs(w, 0, N)
    oc = pipeline.build_layer(K, V, k_mode=w.k_mode, v_mode=w.v_mode, v_bits=w.v_bits, n_cap=n_cap, meta=m,
                              k_bits=w.k_bits or 4, k_group=w.k_group or 32, k_rot=ks, v_rot=vs)
    cache = P.PackedCache(L=1, B=w.B, Hq=w.Hq, Hkv=w.Hkv, n_cap=n_cap,
                          k_mode=P.K_BLOCKGTQ if w.k_mode == "gtq" else P.K_AFFINE,
                          budget_units=w.k_budget_units or 128, k_bits=w.k_bits or 4, k_group=w.k_group or 32,
                          v_mode=P.V_CODEBOOK if w.v_mode == "codebook" else P.V_AFFINE, v_bits=w.v_bits,
                          k_rotation=krot, v_rotation=True)
    if m is not None:
        cache.set_metadata(0, m.bits, m.sigma, m.r)
    if krot:
        cache.set_key_rotation(0, ks)
    cache.set_value_rotation(0, vs)
    T.append_all(cache, 0, K, V, w.dtype, chunks)
    _compare_cache(cache, oc, w)
    ref = pipeline.decode_layer(oc, q)
    qd = T.to_dev(q, w.dtype)
    for ns in (0, 1, 3):
        out = cache.decode_attention(0, qd, n_splits=ns)
        torch.cuda.synchronize()
        e = T.assert_close(out.cpu().numpy(), ref, f"{name} splits={ns}")
        print(f"  splits={ns}: max abs err {e:.2e}", flush=True)
    # one decode step on top: the appended token goes through the rotated quantizer
    kd = T.to_dev(np.transpose(K, (0, 2, 1, 3))[:, -1:], w.dtype)
    vd = T.to_dev(np.transpose(V, (0, 2, 1, 3))[:, -1:], w.dtype)
    cache.n_tokens[0] -= 1
    out = cache.decode_step(0, kd, vd, qd)
    torch.cuda.synchronize()
    T.assert_close(out.cpu().numpy(), ref, f"{name} step")
    _compare_cache(cache, oc, w)


EDGE_CASES = {
    # name: (workload id, overrides, N, n_splits)
    "max_batch_64": (3, {"L": 1, "B": 64, "Hkv": 1, "Hq": 4}, 70, 0),
    "splits_far_beyond_tiles": (2, {"L": 1}, 5 * 64 - 3, 40),
    "one_token_mx": (2, {"L": 1}, 1, 0),
    "one_token_vector": (1, {}, 1, 0),
    "one_token_affine": (4, {"L": 1, "B": 1, "Hkv": 1, "Hq": 4}, 1, 3),
}


@pytest.mark.parametrize("name", list(EDGE_CASES))
def test_decode_edge_cases(name):
    """The largest batch the library takes, splits that own no tile (their partials carry no
    weight in the merge), and a context of a single token (the output is that token's value)."""
    wid, ov, N, ns = EDGE_CASES[name]
    w = synth.reduced(synth.WORKLOADS[wid], **ov)
    print(f"[edge {name}] N={N} B={w.B} Hq={w.Hq} Hkv={w.Hkv} splits={ns}", flush=True)
    n_cap = ((N + 63) // 64) * 64
    m = T.meta(w, 0)
    K, V, q = T.inputs(w, 0, N)
    oc = T.oracle_layer(w, K, V, m, n_cap)
    cache = T.gpu_cache(w, n_cap)
    if m is not None:
        cache.set_metadata(0, m.bits, m.sigma, m.r)
    T.append_all(cache, 0, K, V, w.dtype)
    _compare_cache(cache, oc, w)
    ref = pipeline.decode_layer(oc, q)
    out = cache.decode_attention(0, T.to_dev(q, w.dtype), n_splits=ns).cpu().numpy()
    e = T.assert_close(out, ref, name)
    print(f"  max abs err {e:.2e}", flush=True)


def test_decode_deterministic_and_split_invariant():
    w = synth.reduced(synth.WORKLOADS[2], L=1)
    N = 5000
    m = T.meta(w, 0)
    K, V, q = T.inputs(w, 0, N)
    cache = T.gpu_cache(w, 5120)
    cache.set_metadata(0, m.bits, m.sigma, m.r)
    T.append_all(cache, 0, K, V, w.dtype)
    qd = T.to_dev(q, w.dtype)
    a = cache.decode_attention(0, qd, n_splits=7).cpu().numpy()
    b = cache.decode_attention(0, qd, n_splits=7).cpu().numpy()
    np.testing.assert_array_equal(a, b)
    c = cache.decode_attention(0, qd, n_splits=2).cpu().numpy()
    assert np.max(np.abs(a - c)) < 1e-4


def test_ragged_sequence_lengths():
    """Sequences of one batch with different lengths (host n_tokens per sequence)."""
    w = synth.reduced(synth.WORKLOADS[3], L=1, B=3)
    N = 700
    m = T.meta(w, 0)
    K, V, q = T.inputs(w, 0, N)
    cache = T.gpu_cache(w, 768)
    cache.set_metadata(0, m.bits, m.sigma, m.r)
    T.append_all(cache, 0, K, V, w.dtype)
    lens = [700, 1, 333]
    cache.n_tokens[0, :] = lens
    out = cache.decode_attention(0, T.to_dev(q, w.dtype), n_splits=2).cpu().numpy()
    for b, n in enumerate(lens):
        wb = synth.reduced(w, B=1)
        oc = T.oracle_layer(wb, K[b:b + 1, :, :n], V[b:b + 1, :, :n], m, 768)
        ref = pipeline.decode_layer(oc, q[b:b + 1])
        T.assert_close(out[b:b + 1], ref, f"ragged b={b} n={n}")


def test_errors_on_device_paths():
    w = synth.reduced(synth.WORKLOADS[1], N=64)
    cache = T.gpu_cache(w, 64)
    q = torch.zeros((1, 1, 128), device="cuda")
    with pytest.raises(P.BgtqError) as e:
        cache.decode_attention(0, q, n_splits=1)                  # empty context
    assert e.value.code == P.E_INVALID
    k = torch.zeros((1, 65, 1, 128), device="cuda")
    with pytest.raises(P.BgtqError) as e:
        cache.quantize_append(0, k, k)                             # capacity
    assert e.value.code == P.E_CAPACITY
    assert cache.n_tokens[0, 0] == 0


def test_metadata_widths_validated_and_bounded():
    """set_metadata rejects widths that do not sum to the budget; widths written to the device
    buffer directly (bypassing the binding) never make the quantizer write past a token's record:
    the later tiles of a three-tile cache stay untouched while the first is appended.  (Three
    tiles hold 8 KB per (b, h), so even an unbounded write of 32-dword records would stay inside
    the buffer.)"""
    w = synth.reduced(synth.WORKLOADS[2], L=1)
    cache = T.gpu_cache(w, 192)
    m = T.meta(w, 0)
    bad = m.bits.copy()
    bad[0, int(np.argmax(bad[0] < 8))] += 1                      # one bit over the budget
    with pytest.raises(ValueError):
        cache.set_metadata(0, bad, m.sigma, m.r)
    with pytest.raises(ValueError):
        cache.set_metadata(0, np.full_like(m.bits, 9), m.sigma, m.r)
    cache.set_metadata(0, m.bits, m.sigma, m.r)
    over = np.full((w.Hkv, 64), 8, np.uint8)                      # 1024 bits: far past the 384-bit record
    cache.bits[0].copy_(torch.from_numpy(over))
    K, V, _ = T.inputs(w, 0, 64)
    T.append_all(cache, 0, K, V, w.dtype)
    kc = T.layer_view(cache.k_codes, 1, 0, (w.B, w.Hkv, 3, -1)).cpu().numpy()
    assert np.all(kc[:, :, 1:] == 0), "the quantizer wrote past the first tile"
    assert np.any(kc[:, :, 0] != 0)


FP16_CASES = {
    # name: (workload id, overrides, N, n_splits); 4 and 8 query heads per kv head take the
    # matrix-core kernel, 1 and 2 the vector one
    "g8_splits5": (2, {"L": 1, "B": 2}, 3000, 5),
    "g8_auto_ragged": (2, {"L": 1}, 64 * 7 + 13, 0),
    "g8_one_split_tail": (2, {"L": 1}, 200, 1),
    "g4_auto": (3, {"L": 1, "B": 2}, 2048 + 5, 0),
    "g4_fp32_query": (3, {"L": 1, "B": 1, "dtype": "f32"}, 1000, 3),
    "g1_vector": (1, {}, 1000, 3),
    "g2_vector": (2, {"L": 1, "Hq": 4, "Hkv": 2}, 777, 0),
}


@pytest.mark.parametrize("name", list(FP16_CASES))
def test_fp16_baseline_decode(name):
    wid, ov, N, ns = FP16_CASES[name]
    w = synth.reduced(synth.WORKLOADS[wid], **ov)
    K, V, q = T.inputs(w, 0, N)
    k16 = K.astype(np.float16)
    v16 = V.astype(np.float16)
    ref = pipeline.fp16_decode(k16, v16, q)
    out = P.bgtq_fp16_decode_attention(torch.from_numpy(k16).cuda(), torch.from_numpy(v16).cuda(),
                                       T.to_dev(q, w.dtype), n_splits=ns)
    T.assert_close(out.cpu().numpy(), ref, f"fp16 baseline {name}")


@pytest.mark.parametrize("wid", [1, 3])
def test_block_energy(wid):
    from oracle import energy
    w = synth.WORKLOADS[wid]
    cal = [synth.calibration(w, 0, h) for h in range(w.Hkv)]
    kc = np.stack([c[0] for c in cal], axis=1)                    # [T, Hkv, d]
    qc = np.concatenate([np.transpose(c[1], (1, 0, 2)) for c in cal], axis=1)  # [T, Hq, d]
    sc, sg, rs = P.bgtq_block_energy(T.to_dev(kc, w.dtype), T.to_dev(qc, w.dtype))
    for h in range(w.Hkv):
        ek, eq = energy.block_energy(cal[h][0], cal[h][1])
        np.testing.assert_allclose(sc[h], energy.scores(ek, eq), rtol=1e-12)
        s_o, r_o = energy.sigma_hat(ek)
        assert np.max(np.abs(sg[h].astype(np.float64) / s_o - 1)) <= 2 ** -23


STEP_CASES = {
    # name: (workload id, overrides, prefill tokens, tokens appended per decode step)
    "w2_steps_cross_tile": (2, {"L": 1}, 1022, (1, 1, 1, 3, 1)),
    "w1_from_empty": (1, {}, 0, (1, 1, 62, 1, 1)),
    "w5_ring_evicts": (5, {}, 300, (1, 1, 2, 1)),
    "w4_affine_steps": (4, {"L": 1, "B": 2}, 500 + 11, (1, 1, 1)),
}


@pytest.mark.parametrize("name", list(STEP_CASES))
def test_decode_step_matches_append_then_attend(name):
    """bgtq_decode_step: each step appends its rows and attends the step's query over the grown
    context; every output matches the oracle over the same prefix, and the cache ends bit-exact."""
    wid, ov, n0, steps = STEP_CASES[name]
    w = synth.reduced(synth.WORKLOADS[wid], **ov)
    N = n0 + sum(steps)
    print(f"[step case {name}] prefill={n0} steps={steps} B={w.B} Hq={w.Hq} Hkv={w.Hkv}", flush=True)
    n_cap = ((N + 63) // 64 + 1) * 64
    m = T.meta(w, 0)
    K, V, _ = T.inputs(w, 0, N)
    cache = T.gpu_cache(w, n_cap)
    if m is not None:
        cache.set_metadata(0, m.bits, m.sigma, m.r)
    if n0:
        T.append_all(cache, 0, K[:, :, :n0], V[:, :, :n0], w.dtype)
    kd = T.to_dev(np.transpose(K, (0, 2, 1, 3)), w.dtype)        # [B, N, Hkv, d]
    vd = T.to_dev(np.transpose(V, (0, 2, 1, 3)), w.dtype)
    pos = n0
    for i, n in enumerate(steps):
        q = np.stack([np.concatenate([synth.queries(w, 0, h, b, pos + n) for h in range(w.Hkv)])
                      for b in range(w.B)])
        out = cache.decode_step(0, kd[:, pos:pos + n], vd[:, pos:pos + n], T.to_dev(q, w.dtype),
                                n_splits=(0, 3)[i % 2])
        torch.cuda.synchronize()
        pos += n
        assert (cache.n_tokens[0] == pos).all()
        oc = T.oracle_layer(w, K[:, :, :pos], V[:, :, :pos], m, n_cap)
        e = T.assert_close(out.cpu().numpy(), pipeline.decode_layer(oc, q), f"{name} step {i} (context {pos})")
        print(f"  step {i}: context {pos}, max abs err {e:.2e}", flush=True)
    _compare_cache(cache, oc, w)


FUSED_CASES = {
    # name: (workload id, overrides, prefill tokens, one-token steps, n_splits per step).  One token
    # per sequence on the plan-driven kernel is quantized inside the decode launch; these cover its
    # eight-wave looping kernel (more than 16 tiles per split), affine and 4-bit values, fp16 rows,
    # 4 query heads per kv head with two sequences, and tokens at the last position of a tile and at
    # the first position of a new one.
    "g8_looping_kernel": (2, {"L": 1}, 2046, 3, (1, 2, 1)),
    "g8_affine_values": (2, {"L": 1, "v_mode": "affine"}, 127, 3, (0, 1, 3)),
    "g8_k4v4_f16": (2, {"L": 1, "v_bits": 4, "k_budget_units": 256, "dtype": "f16"}, 190, 3, (0, 2, 1)),
    "g4_two_sequences": (3, {"L": 1, "B": 2}, 1300, 2, (0, 1)),
}


@pytest.mark.parametrize("name", list(FUSED_CASES))
def test_fused_decode_step(name):
    """One-token decode steps that the decode launch appends itself: every output matches the
    oracle over the grown context and the cache ends bit-exact (codes, scales, value streams)."""
    wid, ov, n0, n_steps, splits = FUSED_CASES[name]
    w = synth.reduced(synth.WORKLOADS[wid], **ov)
    N = n0 + n_steps
    print(f"[fused step {name}] prefill={n0} steps={n_steps} B={w.B} Hq={w.Hq} Hkv={w.Hkv}", flush=True)
    n_cap = ((N + 63) // 64 + 1) * 64
    m = T.meta(w, 0)
    K, V, _ = T.inputs(w, 0, N)
    cache = T.gpu_cache(w, n_cap)
    cache.set_metadata(0, m.bits, m.sigma, m.r)
    T.append_all(cache, 0, K[:, :, :n0], V[:, :, :n0], w.dtype)
    kd = T.to_dev(np.transpose(K, (0, 2, 1, 3)), w.dtype)        # [B, N, Hkv, d]
    vd = T.to_dev(np.transpose(V, (0, 2, 1, 3)), w.dtype)
    pos = n0
    for i in range(n_steps):
        q = np.stack([np.concatenate([synth.queries(w, 0, h, b, pos + 1) for h in range(w.Hkv)])
                      for b in range(w.B)])
        out = cache.decode_step(0, kd[:, pos:pos + 1], vd[:, pos:pos + 1], T.to_dev(q, w.dtype), n_splits=splits[i])
        torch.cuda.synchronize()
        pos += 1
        assert (cache.n_tokens[0] == pos).all()
        oc = T.oracle_layer(w, K[:, :, :pos], V[:, :, :pos], m, n_cap)
        e = T.assert_close(out.cpu().numpy(), pipeline.decode_layer(oc, q), f"{name} step {i} (context {pos})")
        print(f"  step {i}: context {pos}, splits {splits[i]}, max abs err {e:.2e}", flush=True)
    _compare_cache(cache, oc, w)


FEW_CASES = {
    # name: (workload id, overrides, N, chunk sizes).  Short appends take the one-token-per-wave
    # kernel (at most 16 positions per sequence for 16-bit rows with Block-GTQ keys and codebook
    # values, at most 64 otherwise); every format it covers, appended a few tokens at a time
    # (including chunks that straddle a tile boundary, and longer chunks that take the bulk kernel).
    "gtq_v3_g8": (2, {"L": 1}, 150, (1, 1, 5, 16, 17, 1, 60, 1, 3, 40, 1)),
    "gtq_v2_b2": (3, {"L": 1, "B": 2}, 90, (1, 2, 3, 16, 1, 7, 60)),
    "gtq_v4_k4": (2, {"L": 1, "v_bits": 4, "k_budget_units": 256}, 70, (1, 13, 1, 16, 39)),
    "gtq_v1": (1, {"v_bits": 1}, 66, (1, 1, 62, 2)),
    "affine_g32_v2": (4, {"L": 1, "B": 2}, 80, (1, 1, 14, 48, 16)),
    "affine_g64_codebook_v3": (4, {"L": 1, "B": 1, "k_group": 64, "v_mode": "codebook", "v_bits": 3}, 70,
                               (2, 16, 16, 16, 20)),
    "affine_g128_k8": (4, {"L": 1, "B": 1, "k_group": 128, "k_bits": 8}, 40, (1, 3, 36)),
    "ring_evicts_few": (5, {}, 300, (100, 156, 1, 1, 16, 2, 24)),
}


@pytest.mark.parametrize("name", list(FEW_CASES))
def test_few_token_appends_bit_exact(name):
    wid, ov, N, chunks = FEW_CASES[name]
    w = synth.reduced(synth.WORKLOADS[wid], **ov)
    print(f"[few case {name}] N={N} chunks={chunks}", flush=True)
    n_cap = ((N + 63) // 64 + 1) * 64
    m = T.meta(w, 0)
    K, V, q = T.inputs(w, 0, N)
    oc = T.oracle_layer(w, K, V, m, n_cap)
    cache = T.gpu_cache(w, n_cap)
    if m is not None:
        cache.set_metadata(0, m.bits, m.sigma, m.r)
    T.append_all(cache, 0, K, V, w.dtype, chunks)
    _compare_cache(cache, oc, w)
    if name in ("gtq_v1", "affine_g128_k8"):   # formats the quantizer writes but no decode kernel reads
        return
    out = cache.decode_attention(0, T.to_dev(q, w.dtype))
    torch.cuda.synchronize()
    T.assert_close(out.cpu().numpy(), pipeline.decode_layer(oc, q), name)


BULK_CASES = {
    # name: (workload id, overrides, N, chunk sizes, decoded).  Appends of more than 64 positions
    # per sequence take the bulk quantizer; 16-bit rows with Block-GTQ keys and codebook values take
    # the kernels that hold each row in registers.  fp16 and bf16 rows, record sizes from 1 to 32
    # dwords, value widths 1 to 4, chunks that start inside a tile (the streams of the tile's
    # earlier tokens keep their bits) and two sequences.  Formats no decode kernel reads compare
    # the packed store only.
    "gtq_f16_k3v3": (2, {"L": 1, "dtype": "f16"}, 1000 + 21, (130, 77, None), True),
    "gtq_bf16_v1_r1": (2, {"L": 1, "v_bits": 1, "k_budget_units": 16}, 700 + 5, (65, 200, None), False),
    "gtq_bf16_v4_r32": (2, {"L": 1, "v_bits": 4, "k_budget_units": 512}, 600 + 3, (100, None), False),
    "gtq_f16_v2_r8_b2": (3, {"L": 1, "B": 2, "dtype": "f16"}, 900 + 9, (333, 65, None), True),
    "gtq_bf16_v3_r16": (2, {"L": 1, "v_bits": 3, "k_budget_units": 256}, 400 + 1, (None,), True),
}


@pytest.mark.parametrize("name", list(BULK_CASES))
def test_bulk_quantize_bit_exact(name):
    wid, ov, N, chunks, decoded = BULK_CASES[name]
    w = synth.reduced(synth.WORKLOADS[wid], **ov)
    print(f"[bulk case {name}] N={N} chunks={chunks}", flush=True)
    n_cap = ((N + 63) // 64 + 1) * 64
    m = T.meta(w, 0)
    K, V, q = T.inputs(w, 0, N)
    oc = T.oracle_layer(w, K, V, m, n_cap)
    cache = T.gpu_cache(w, n_cap)
    cache.set_metadata(0, m.bits, m.sigma, m.r)
    T.append_all(cache, 0, K, V, w.dtype, chunks)
    _compare_cache(cache, oc, w)
    if decoded:
        out = cache.decode_attention(0, T.to_dev(q, w.dtype))
        torch.cuda.synchronize()
        T.assert_close(out.cpu().numpy(), pipeline.decode_layer(oc, q), name)


def test_decode_step_ragged_lengths():
    """Decode steps on sequences of different lengths: each sequence appends at its own position
    (other tiles, over bits of an earlier, longer fill that the decode must ignore)."""
    w = synth.reduced(synth.WORKLOADS[3], L=1, B=3)
    N = 700
    m = T.meta(w, 0)
    K, V, _ = T.inputs(w, 0, N)
    cache = T.gpu_cache(w, 768)
    cache.set_metadata(0, m.bits, m.sigma, m.r)
    T.append_all(cache, 0, K, V, w.dtype)
    lens = np.array([640, 1, 333])
    cache.n_tokens[0, :] = lens
    for step in range(3):
        kn = np.stack([K[b, :, lens[b]] for b in range(w.B)])[:, None]      # [B, 1, Hkv, d]
        vn = np.stack([V[b, :, lens[b]] for b in range(w.B)])[:, None]
        q = np.stack([np.concatenate([synth.queries(w, 0, h, b, int(lens[b]) + 1) for h in range(w.Hkv)])
                      for b in range(w.B)])
        out = cache.decode_step(0, T.to_dev(kn, w.dtype), T.to_dev(vn, w.dtype), T.to_dev(q, w.dtype),
                                n_splits=(0, 2, 5)[step]).cpu().numpy()
        lens = lens + 1
        assert (cache.n_tokens[0] == lens).all()
        for b in range(w.B):
            wb = synth.reduced(w, B=1)
            oc = T.oracle_layer(wb, K[b:b + 1, :, :lens[b]], V[b:b + 1, :, :lens[b]], m, 768)
            T.assert_close(out[b:b + 1], pipeline.decode_layer(oc, q[b:b + 1]), f"step {step} b={b} n={lens[b]}")


@pytest.mark.parametrize("wid,N", [(2, 1500 + 7), (5, 200)])
def test_graph_replays_match_eager(wid, N):
    """Decode and the append-then-attend step captured in a HIP graph: every replay (eager work and
    synchronizations between replays) equals the eager result bit for bit, and the cache bytes
    stay those the eager step wrote.  (A replayed step rewrites its position with the same row; with
    the fp16 window the context stays inside it, since a step that evicts reads the ring slot it
    then overwrites and so is not the same step twice.)"""
    w = synth.reduced(synth.WORKLOADS[wid], L=1) if wid != 5 else synth.WORKLOADS[5]
    m = T.meta(w, 0)
    K, V, q = T.inputs(w, 0, N)
    cache = T.gpu_cache(w, ((N + 63) // 64 + 1) * 64)
    cache.set_metadata(0, m.bits, m.sigma, m.r)
    T.append_all(cache, 0, K[:, :, :N - 1], V[:, :, :N - 1], w.dtype)
    kd = T.to_dev(np.transpose(K[:, :, N - 1:], (0, 2, 1, 3)), w.dtype)
    vd = T.to_dev(np.transpose(V[:, :, N - 1:], (0, 2, 1, 3)), w.dtype)
    qd = T.to_dev(q, w.dtype)
    ws = cache.workspace()
    out_step = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    cache.decode_step(0, kd, vd, qd, out=out_step, ws=ws)
    eager_step = out_step.clone()
    eager_dec = cache.decode_attention(0, qd, ws=ws).clone()
    bufs = lambda: [t for t in (cache.k_codes, cache.v_codes, cache.k_scale, cache.v_scale, cache.recent_k,
                                cache.recent_v) if t is not None]
    snap = [t.clone() for t in bufs()]
    torch.cuda.synchronize()
    out_dec = torch.empty_like(out_step)
    g_dec, g_step = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_dec):
        cache.decode_attention(0, qd, out=out_dec, ws=ws)
    cache.n_tokens[0] -= 1                       # the captured step re-appends position N - 1
    with torch.cuda.graph(g_step):
        cache.decode_step(0, kd, vd, qd, out=out_step, ws=ws)
    assert (cache.n_tokens[0] == N).all()
    for r in range(3):
        out_step.zero_()
        out_dec.zero_()
        g_step.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out_step.cpu().numpy(), eager_step.cpu().numpy(), f"step replay {r}")
        other = cache.decode_attention(0, qd * 0.5, ws=torch.empty_like(ws))   # eager work between replays
        g_dec.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out_dec.cpu().numpy(), eager_dec.cpu().numpy(), f"decode replay {r}")
        assert torch.isfinite(other).all()
        for a, b in zip(snap, bufs()):
            assert torch.equal(a, b), f"cache bytes changed on replay {r}"


def test_decode_step_rotated_keys():
    """Decode steps with rotated affine keys (their appends take the tile kernel): every step's
    output matches the oracle over the same prefix, and the cache ends bit-exact."""
    w = synth.reduced(synth.WORKLOADS[4], L=1, B=2)
    n0, steps = 300 + 5, (1, 2, 1)
    N = n0 + sum(steps)
    n_cap = ((N + 63) // 64 + 1) * 64
    signs = np.where(np.random.default_rng(47).random((w.Hkv, 128)) < 0.5, -1.0, 1.0)
    K, V, _ = T.inputs(w, 0, N)
    cache = P.PackedCache(L=1, B=w.B, Hq=w.Hq, Hkv=w.Hkv, n_cap=n_cap, k_mode=P.K_AFFINE, k_bits=w.k_bits,
                          k_group=w.k_group, v_mode=P.V_AFFINE, v_bits=w.v_bits, k_rotation=True)
    cache.set_key_rotation(0, signs)
    T.append_all(cache, 0, K[:, :, :n0], V[:, :, :n0], w.dtype)
    kd = T.to_dev(np.transpose(K, (0, 2, 1, 3)), w.dtype)
    vd = T.to_dev(np.transpose(V, (0, 2, 1, 3)), w.dtype)
    pos = n0
    for i, n in enumerate(steps):
        q = np.stack([np.concatenate([synth.queries(w, 0, h, b, pos + n) for h in range(w.Hkv)])
                      for b in range(w.B)])
        out = cache.decode_step(0, kd[:, pos:pos + n], vd[:, pos:pos + n], T.to_dev(q, w.dtype)).cpu().numpy()
        pos += n
        oc = pipeline.build_layer(K[:, :, :pos], V[:, :, :pos], k_mode="affine", v_mode="affine", v_bits=w.v_bits,
                                  n_cap=n_cap, k_bits=w.k_bits, k_group=w.k_group, k_rot=signs)
        T.assert_close(out, pipeline.decode_layer(oc, q), f"rotated step {i} (context {pos})")
    _compare_cache(cache, oc, w)


PREFILL_CASES = {
    # name: (workload id, overrides, W, prompt tokens): Block-GTQ at 8 and 4 query heads per kv head
    # (two sequences), fp32 rows at one (their fp16 rounding matters), affine K4V2
    "g8_w4": (2, {"L": 1, "B": 1}, 4, 700),
    "g4_b2_w8": (3, {"L": 1, "B": 2}, 8, 1500),
    "g1_fp32_w2": (1, {}, 2, 300),
    "affine_b2_w16": (4, {"L": 1, "B": 2}, 16, 1100),
}


@pytest.mark.parametrize("name", list(PREFILL_CASES))
def test_logquant_prefill_matches_oracle(name):
    """LogQuant's filter over a whole prompt in one call: the packed store equals the oracle's
    store of the leaving tokens (fp16-rounded, as they leave the store) in leaving order, bit-exact;
    the high-precision store holds the kept positions' fp16 rows in position order; decode matches
    the oracle; and a cache fed the same prompt token by token holds the same packed bytes."""
    from oracle import logquant as lq
    wid, ov, W, N = PREFILL_CASES[name]
    w = synth.reduced(synth.WORKLOADS[wid], **ov)
    print(f"[prefill {name}] W={W} N={N} B={w.B} Hq={w.Hq} Hkv={w.Hkv}", flush=True)
    kept, left = lq.select(N, W)
    n_cap, R = (len(left) + 63) // 64 * 64 + 64, 3 * W
    m = T.meta(w, 0)
    K, V, _ = T.inputs(w, 0, N)
    caches = []
    for _ in range(2):
        c = P.PackedCache(L=1, B=w.B, Hq=w.Hq, Hkv=w.Hkv, n_cap=n_cap,
                          k_mode=P.K_BLOCKGTQ if w.k_mode == "gtq" else P.K_AFFINE,
                          budget_units=w.k_budget_units or 128, k_bits=w.k_bits or 4, k_group=w.k_group or 32,
                          v_mode=P.V_CODEBOOK if w.v_mode == "codebook" else P.V_AFFINE, v_bits=w.v_bits,
                          logquant_w=W)
        if m is not None:
            c.set_metadata(0, m.bits, m.sigma, m.r)
        caches.append(c)
    cache, ref_cache = caches
    kd = T.to_dev(np.transpose(K, (0, 2, 1, 3)), w.dtype)
    vd = T.to_dev(np.transpose(V, (0, 2, 1, 3)), w.dtype)
    cache.logquant_prefill(0, kd, vd)
    torch.cuda.synchronize()
    assert (cache.n_tokens[0] == N).all() and (cache.n_hp[0] == len(kept)).all()
    k16 = K[:, :, left].astype(np.float16).astype(np.float32)
    v16 = V[:, :, left].astype(np.float16).astype(np.float32)
    oc = pipeline.build_layer(k16, v16, k_mode=w.k_mode, v_mode=w.v_mode, v_bits=w.v_bits, n_cap=n_cap, meta=m,
                              k_bits=w.k_bits or 4, k_group=w.k_group or 32)
    _compare_cache(cache, oc, w)
    rk = T.layer_view(cache.recent_k, 1, 0, (w.B, w.Hkv, R, 128)).cpu().numpy()
    rv = T.layer_view(cache.recent_v, 1, 0, (w.B, w.Hkv, R, 128)).cpu().numpy()
    for b in range(w.B):
        assert cache.hp_pos[0, b, :len(kept)].tolist() == kept
        np.testing.assert_array_equal(rk[b, :, :len(kept)].view(np.uint16),
                                      K[b][:, kept].astype(np.float16).view(np.uint16), f"store k b={b}")
        np.testing.assert_array_equal(rv[b, :, :len(kept)].view(np.uint16),
                                      V[b][:, kept].astype(np.float16).view(np.uint16), f"store v b={b}")
    oc.recent_k = K[:, :, kept].astype(np.float16)
    oc.recent_v = V[:, :, kept].astype(np.float16)
    oc.n_recent_valid = len(kept)
    q = np.stack([np.concatenate([synth.queries(w, 0, h, b, N) for h in range(w.Hkv)]) for b in range(w.B)])
    out = cache.decode_attention(0, T.to_dev(q, w.dtype)).cpu().numpy()
    e = T.assert_close(out, pipeline.decode_layer(oc, q), f"prefill {name}")
    print(f"  {len(left)} packed + {len(kept)} fp16, max abs err {e:.2e}", flush=True)
    for p in range(N):
        ref_cache.logquant_append(0, kd[:, p:p + 1], vd[:, p:p + 1])
    torch.cuda.synchronize()
    for name_ in ("k_codes", "v_codes", "k_scale", "v_scale", "k_zero", "v_zero"):
        a, r = getattr(cache, name_), getattr(ref_cache, name_)
        if a is not None:
            assert torch.equal(a, r), f"{name_}: prefill and token-by-token appends differ"


# W > 16 sends a halving's W leaving rows through the bulk quantizer (16-bit store rows, appended
# mid-tile for W = 24), smaller W through the one-token-per-wave kernel
@pytest.mark.parametrize("wid,W,N", [(2, 4, 70), (3, 8, 100), (1, 2, 40), (4, 4, 60), (2, 32, 140), (3, 24, 110)])
def test_logquant_appends_match_oracle(wid, W, N):
    """LogQuant's log-based filter through the device: after token-by-token appends, the packed
    store equals the oracle's store of the leaving tokens in leaving order (bit-exact), the
    high-precision store holds exactly the kept positions' fp16 rows, and decode matches the
    oracle over the union of both."""
    from oracle import logquant as lq
    ov = {"L": 1, "B": 2} if wid == 3 else ({} if wid == 1 else {"L": 1, "B": 1})
    w = synth.reduced(synth.WORKLOADS[wid], **ov)
    print(f"[logquant {wid}] W={W} N={N} B={w.B} Hq={w.Hq} Hkv={w.Hkv} keys={w.k_mode}", flush=True)
    n_cap, R = 128, 3 * W
    m = T.meta(w, 0)
    K, V, _ = T.inputs(w, 0, N)
    cache = P.PackedCache(L=1, B=w.B, Hq=w.Hq, Hkv=w.Hkv, n_cap=n_cap,
                          k_mode=P.K_BLOCKGTQ if w.k_mode == "gtq" else P.K_AFFINE,
                          budget_units=w.k_budget_units or 128, k_bits=w.k_bits or 4, k_group=w.k_group or 32,
                          v_mode=P.V_CODEBOOK if w.v_mode == "codebook" else P.V_AFFINE, v_bits=w.v_bits,
                          logquant_w=W)
    if m is not None:
        cache.set_metadata(0, m.bits, m.sigma, m.r)
    kd = T.to_dev(np.transpose(K, (0, 2, 1, 3)), w.dtype)
    vd = T.to_dev(np.transpose(V, (0, 2, 1, 3)), w.dtype)
    checks = {3 * W + 1, 3 * W + W // 2 + 7, N}
    for p in range(N):
        cache.logquant_append(0, kd[:, p:p + 1], vd[:, p:p + 1])
        if p + 1 not in checks:
            continue
        torch.cuda.synchronize()
        kept, left = lq.select(p + 1, W)
        assert (cache.n_tokens[0] == p + 1).all() and (cache.n_hp[0] == len(kept)).all()
        # every token passes through the fp16 store first, so the packed rows are its fp16 values
        k16 = K[:, :, left].astype(np.float16).astype(np.float32)
        v16 = V[:, :, left].astype(np.float16).astype(np.float32)
        oc = pipeline.build_layer(k16, v16, k_mode=w.k_mode, v_mode=w.v_mode, v_bits=w.v_bits, n_cap=n_cap, meta=m,
                                  k_bits=w.k_bits or 4, k_group=w.k_group or 32)
        _compare_cache(cache, oc, w)
        rk = T.layer_view(cache.recent_k, 1, 0, (w.B, w.Hkv, R, 128)).cpu().numpy()
        rv = T.layer_view(cache.recent_v, 1, 0, (w.B, w.Hkv, R, 128)).cpu().numpy()
        for b in range(w.B):
            held = cache.hp_pos[0, b, :len(kept)]
            assert sorted(held.tolist()) == kept
            np.testing.assert_array_equal(rk[b, :, :len(kept)].view(np.uint16),
                                          K[b][:, held].astype(np.float16).view(np.uint16), f"store k b={b}")
            np.testing.assert_array_equal(rv[b, :, :len(kept)].view(np.uint16),
                                          V[b][:, held].astype(np.float16).view(np.uint16), f"store v b={b}")
        oc.recent_k = K[:, :, kept].astype(np.float16)
        oc.recent_v = V[:, :, kept].astype(np.float16)
        oc.n_recent_valid = len(kept)
        q = np.stack([np.concatenate([synth.queries(w, 0, h, b, p + 1) for h in range(w.Hkv)]) for b in range(w.B)])
        out = cache.decode_attention(0, T.to_dev(q, w.dtype)).cpu().numpy()
        e = T.assert_close(out, pipeline.decode_layer(oc, q), f"logquant context {p + 1}")
        print(f"  context {p + 1}: {len(left)} packed + {len(kept)} fp16, max abs err {e:.2e}", flush=True)
