"""Seeded synthetic inputs for the five decode workloads.

Shared by the tests, the bench and the smoke check.  This module draws numbers and
shapes them; it contains none of the method's arithmetic (no energy, allocation,
quantization, packing or attention).  The random numbers come from NumPy's PCG64 seeded
by ``SeedSequence([workload, layer, kv_head, batch, stream])``.

Key/query model (Block-GTQ page, abstract: keys under RoPE decompose into 2-D frequency
blocks): per (layer, kv head) each RoPE block i = coordinates (2i, 2i+1) has a scale
sigma_i drawn log-uniform in [0.05, 8].  Pre-RoPE keys and queries are N(0, sigma_i^2)
per coordinate; some workloads scale the keys of two randomly chosen blocks by 20
("outlier blocks").  RoPE (interleaved pairs, frequency theta^(-2i/d)) is applied in
float64 at positions 0..N-1 for cached keys and at position N for the decode query, then
the result is rounded to the activation dtype.  Values are N(0, 1).
"""
from __future__ import annotations

import dataclasses
import numpy as np

STREAM_SIGMA, STREAM_OUTLIER, STREAM_K, STREAM_V, STREAM_Q, STREAM_KCAL, STREAM_QCAL = range(7)


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    L: int
    Hq: int
    Hkv: int
    N: int
    B: int
    dtype: str            # "f32" | "f16" | "bf16"
    theta: float
    k_mode: str           # "gtq" (per-block widths from the greedy) | "affine" (uniform groups)
    k_budget_units: int   # gtq: sum of per-coordinate widths over the 64 blocks
    k_bits: int           # affine: bits per key coordinate
    k_group: int          # affine: coordinates per (scale, zero) group
    v_mode: str           # "codebook" | "affine"
    v_bits: int
    v_group: int
    t_cal: int
    outliers: int
    n_recent: int
    d: int = 128

    @property
    def g(self) -> int:
        return self.Hq // self.Hkv


WORKLOADS = {
    1: Workload(1, "1 layer, 1q/1kv head, d=128, N=4096, B=1, K2V2, fp32", 1, 1, 1, 4096, 1, "f32",
                1e4, "gtq", 128, 0, 0, "codebook", 2, 128, 512, 0, 0),
    2: Workload(2, "Qwen2.5-3B shape: 36 layers, 16q/2kv, d=128, N=131072, B=1, K3V3, bf16", 36, 16, 2,
                131072, 1, "bf16", 1e6, "gtq", 192, 0, 0, "codebook", 3, 128, 512, 2, 0),
    3: Workload(3, "Llama-3.1-8B shape: 32 layers, 32q/8kv, d=128, N=32768, B=8, K2V2, bf16", 32, 32, 8,
                32768, 8, "bf16", 5e5, "gtq", 128, 0, 0, "codebook", 2, 128, 1024, 0, 0),
    4: Workload(4, "Llama-3.1-8B shape: 32 layers, 32q/8kv, d=128, N=65536, B=2, K4 affine g32 / V2 affine g128, bf16",
                32, 32, 8, 65536, 2, "bf16", 5e5, "affine", 0, 4, 32, "affine", 2, 128, 0, 0, 0),
    5: Workload(5, "Qwen2.5-3B shape: 1 layer, 16q/2kv, d=128, N=524288 (last 256 fp16), B=1, K3V2, bf16", 1, 16, 2,
                524288, 1, "bf16", 1e6, "gtq", 192, 0, 0, "codebook", 2, 128, 512, 2, 256),
}


def rng(wid: int, layer: int, kv_head: int, batch: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([wid, layer, kv_head, batch, stream])))


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to the activation dtype; returned as float32 holding exact values."""
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "f16":
        return x.astype(np.float16).astype(np.float32)
    if dtype == "bf16":
        f = x.astype(np.float32)  # f64 -> f32 (RN), then RNE to 8 significant bits
        u = f.view(np.uint32).astype(np.uint64)
        lsb = (u >> 16) & 1
        u = (u + 0x7FFF + lsb) >> 16 << 16
        return (u & 0xFFFFFFFF).astype(np.uint32).view(np.float32)
    raise ValueError(dtype)


def block_sigmas(w: Workload, layer: int, kv_head: int):
    """(sigma_q[64], sigma_k[64]) for one (layer, kv head): log-uniform [0.05, 8]; keys of
    ``w.outliers`` blocks scaled by 20."""
    nb = w.d // 2
    s = np.exp(rng(w.wid, layer, kv_head, 0, STREAM_SIGMA).uniform(np.log(0.05), np.log(8.0), nb))
    sk = s.copy()
    if w.outliers:
        idx = rng(w.wid, layer, kv_head, 0, STREAM_OUTLIER).choice(nb, w.outliers, replace=False)
        sk[idx] *= 20.0
    return s, sk


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Interleaved rotary embedding in float64: block i = (2i, 2i+1) rotated by pos*theta^(-2i/d)."""
    d = x.shape[-1]
    freq = theta ** (-np.arange(0, d, 2, dtype=np.float64) / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * freq
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x, dtype=np.float64)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def keys(w: Workload, layer: int, kv_head: int, batch: int, n: int, start: int = 0) -> np.ndarray:
    """Post-RoPE cached keys for positions start..start+n-1, float32 holding dtype-exact values."""
    _, sk = block_sigmas(w, layer, kv_head)
    g = rng(w.wid, layer, kv_head, batch, STREAM_K)
    if start:
        g.standard_normal((start, w.d))  # keep the stream position-stable
    z = g.standard_normal((n, w.d)) * np.repeat(sk, 2)
    return round_to_dtype(rope(z, np.arange(start, start + n), w.theta), w.dtype)


def values(w: Workload, layer: int, kv_head: int, batch: int, n: int, start: int = 0) -> np.ndarray:
    g = rng(w.wid, layer, kv_head, batch, STREAM_V)
    if start:
        g.standard_normal((start, w.d))
    return round_to_dtype(g.standard_normal((n, w.d)), w.dtype)


def queries(w: Workload, layer: int, kv_head: int, batch: int, pos: int) -> np.ndarray:
    """[g, d] decode queries of the kv head's group at position ``pos``."""
    sq, _ = block_sigmas(w, layer, kv_head)
    z = rng(w.wid, layer, kv_head, batch, STREAM_Q).standard_normal((w.g, w.d)) * np.repeat(sq, 2)
    return round_to_dtype(rope(z, np.full(w.g, pos), w.theta), w.dtype)


def calibration(w: Workload, layer: int, kv_head: int):
    """(k_cal [T, d], q_cal [g, T, d]) post-RoPE at positions 0..T-1."""
    sq, sk = block_sigmas(w, layer, kv_head)
    T = w.t_cal
    pos = np.arange(T)
    kc = rng(w.wid, layer, kv_head, 0, STREAM_KCAL).standard_normal((T, w.d)) * np.repeat(sk, 2)
    qc = rng(w.wid, layer, kv_head, 0, STREAM_QCAL).standard_normal((w.g, T, w.d)) * np.repeat(sq, 2)
    return (round_to_dtype(rope(kc, pos, w.theta), w.dtype),
            round_to_dtype(rope(qc, np.broadcast_to(pos, (w.g, T)), w.theta), w.dtype))


def reduced(w: Workload, **kw) -> Workload:
    """The same workload with some sizes replaced (parity tests at oracle-friendly sizes)."""
    return dataclasses.replace(w, **kw)
