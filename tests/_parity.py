"""Shared set-up for GPU parity tests: seeded inputs -> (oracle layer cache, GPU PackedCache)."""
from __future__ import annotations

import numpy as np

import synth
from oracle import pipeline

TOL_ABS, TOL_REL = 2e-3, 1e-3


def torch_dtype(name):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[name]


def inputs(w: synth.Workload, layer: int, N: int, bh=None):
    """K, V float32 [B, Hkv, N, d] and q [B, Hq, d] (dtype-exact values)."""
    K = np.zeros((w.B, w.Hkv, N, w.d), np.float32)
    V = np.zeros_like(K)
    q = np.zeros((w.B, w.Hq, w.d), np.float32)
    for b in range(w.B):
        for h in range(w.Hkv):
            if bh is not None and (b, h) not in bh:
                continue
            K[b, h] = synth.keys(w, layer, h, b, N)
            V[b, h] = synth.values(w, layer, h, b, N)
            q[b, h * w.g:(h + 1) * w.g] = synth.queries(w, layer, h, b, N)
    return K, V, q


def meta(w: synth.Workload, layer: int):
    if w.k_mode != "gtq":
        return None
    cal = [synth.calibration(w, layer, h) for h in range(w.Hkv)]
    return pipeline.calibrate([c[0] for c in cal], [c[1] for c in cal], w.k_budget_units)


def oracle_layer(w, K, V, m, n_cap):
    return pipeline.build_layer(K, V, k_mode=w.k_mode, v_mode=w.v_mode, v_bits=w.v_bits, n_cap=n_cap, meta=m,
                                k_bits=w.k_bits or 4, k_group=w.k_group or 32, n_recent=w.n_recent)


def gpu_cache(w, n_cap, L=1):
    import packed_cache_decode_block_amd as P
    return P.PackedCache(L=L, B=w.B, Hq=w.Hq, Hkv=w.Hkv, n_cap=n_cap,
                         k_mode=P.K_BLOCKGTQ if w.k_mode == "gtq" else P.K_AFFINE,
                         budget_units=w.k_budget_units or 128, k_bits=w.k_bits or 4, k_group=w.k_group or 32,
                         v_mode=P.V_CODEBOOK if w.v_mode == "codebook" else P.V_AFFINE, v_bits=w.v_bits,
                         n_recent=w.n_recent)


def to_dev(x, dtype_name):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(torch_dtype(dtype_name))


def append_all(cache, layer, K, V, dtype_name, chunks=(None,)):
    """Append K, V [B, Hkv, N, d] in the given chunk sizes (None = the rest)."""
    import torch
    N = K.shape[2]
    kd = to_dev(np.transpose(K, (0, 2, 1, 3)), dtype_name)   # [B, N, Hkv, d]
    vd = to_dev(np.transpose(V, (0, 2, 1, 3)), dtype_name)
    pos = 0
    for c in chunks:
        n = N - pos if c is None else min(c, N - pos)
        if n <= 0:
            break
        cache.quantize_append(layer, kd[:, pos:pos + n], vd[:, pos:pos + n])
        pos += n
    if pos < N:
        cache.quantize_append(layer, kd[:, pos:], vd[:, pos:])
    torch.cuda.synchronize()


def layer_view(t, L, layer, shape):
    """Slice one layer out of a layer-major flat buffer and reshape."""
    n = t.numel() // L
    return t[layer * n:(layer + 1) * n].reshape(shape)


def assert_close(got, ref, what=""):
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref)
    lim = TOL_ABS + TOL_REL * np.abs(ref)
    bad = err > lim
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside 2e-3 + 1e-3|ref|; max abs err "
                           f"{err.max():.3e} at {np.unravel_index(err.argmax(), err.shape)}")
    return float(err.max())
