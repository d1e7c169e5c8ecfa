"""The synthetic workload recipe of ``synth`` drawn with torch on a GPU (for full-size benches).

Same distributions as the NumPy generator (per-block log-uniform sigma from ``synth.block_sigmas``,
N(0, sigma^2) keys/queries, x20 outlier key blocks, N(0,1) values, interleaved RoPE in float64,
rounding to the activation dtype); the random stream is torch's Philox seeded from the same
(workload, layer, kv head, batch, stream) tuple, so values differ from the NumPy draw.
"""
from __future__ import annotations

import numpy as np
import torch

from . import STREAM_K, STREAM_Q, STREAM_V, Workload, block_sigmas

_TD = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _gen(w: Workload, layer: int, kv_head: int, batch: int, stream: int, device) -> torch.Generator:
    seed = int(np.random.SeedSequence([w.wid, layer, kv_head, batch, stream]).generate_state(1, np.uint64)[0])
    g = torch.Generator(device=device)
    g.manual_seed(seed & 0x7FFFFFFFFFFFFFFF)
    return g


def _rope(x: torch.Tensor, pos: torch.Tensor, theta: float) -> torch.Tensor:
    d = x.shape[-1]
    freq = theta ** (-torch.arange(0, d, 2, dtype=torch.float64, device=x.device) / d)
    ang = pos.to(torch.float64)[..., None] * freq
    c, s = torch.cos(ang), torch.sin(ang)
    a, b = x[..., 0::2], x[..., 1::2]
    out = torch.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def keys(w: Workload, layer: int, kv_head: int, batch: int, n: int, device="cuda") -> torch.Tensor:
    """[n, d] post-RoPE keys in the activation dtype."""
    _, sk = block_sigmas(w, layer, kv_head)
    sig = torch.from_numpy(np.repeat(sk, 2)).to(device)
    z = torch.randn((n, w.d), generator=_gen(w, layer, kv_head, batch, STREAM_K, device), dtype=torch.float64,
                    device=device) * sig
    return _rope(z, torch.arange(n, device=device), w.theta).to(torch.float32).to(_TD[w.dtype])


def values(w: Workload, layer: int, kv_head: int, batch: int, n: int, device="cuda") -> torch.Tensor:
    z = torch.randn((n, w.d), generator=_gen(w, layer, kv_head, batch, STREAM_V, device), dtype=torch.float64,
                    device=device)
    return z.to(torch.float32).to(_TD[w.dtype])


def queries(w: Workload, layer: int, kv_head: int, batch: int, pos: int, device="cuda") -> torch.Tensor:
    sq, _ = block_sigmas(w, layer, kv_head)
    sig = torch.from_numpy(np.repeat(sq, 2)).to(device)
    z = torch.randn((w.g, w.d), generator=_gen(w, layer, kv_head, batch, STREAM_Q, device), dtype=torch.float64,
                    device=device) * sig
    return _rope(z, torch.full((w.g,), pos, device=device), w.theta).to(torch.float32).to(_TD[w.dtype])
