"""GPU parity at full workload sizes, in the launch configuration the bench times.

One layer of every Block-GTQ / affine workload at its full context length, batch and head counts,
decoded with the automatic split count.  Inputs come from the torch recipe of the synthetic
generator on the device (the same inputs the bench uses); the oracle quantizes and decodes
sampled (batch, kv head) pairs of those inputs (both kv heads for the two-kv-head shapes).
Bit-exact: packed codes, scales and the fp16 ring of each sampled pair.  Outputs: the usual
|gpu - ref| <= 2e-3 + 1e-3*|ref| for the query heads of each sampled pair.
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

from synth import gpu as sg  # noqa: E402

SAMPLES = {2: [(0, 0), (0, 1)], 3: [(0, 0), (7, 5)], 4: [(1, 6)], 5: [(0, 1)]}


def _pair_meta(m, h):
    if m is None:
        return None
    return pipeline.LayerMeta(m.bits[h:h + 1], m.sigma[h:h + 1], m.r[h:h + 1], m.scores[h:h + 1])


@pytest.mark.parametrize("wid", sorted(SAMPLES))
def test_full_size_layer(wid):
    w = synth.reduced(synth.WORKLOADS[wid], L=1)
    N, g = w.N, w.g
    print(f"[full size] workload {wid}: N={N} B={w.B} Hq={w.Hq} Hkv={w.Hkv} pairs={SAMPLES[wid]}", flush=True)
    n_cap = (N - min(N, w.n_recent) + 63) // 64 * 64
    m = T.meta(w, 0)
    cache = T.gpu_cache(w, n_cap)
    if m is not None:
        cache.set_metadata(0, m.bits, m.sigma, m.r)
    kk = torch.stack([torch.stack([sg.keys(w, 0, h, b, N) for h in range(w.Hkv)], dim=1) for b in range(w.B)])
    vv = torch.stack([torch.stack([sg.values(w, 0, h, b, N) for h in range(w.Hkv)], dim=1) for b in range(w.B)])
    q = torch.stack([torch.cat([sg.queries(w, 0, h, b, N) for h in range(w.Hkv)]) for b in range(w.B)])
    cache.quantize_append(0, kk, vv)
    out = cache.decode_attention(0, q, n_splits=0).cpu().numpy()
    torch.cuda.synchronize()
    wb = synth.reduced(w, B=1, Hkv=1, Hq=g)
    for b, h in SAMPLES[wid]:
        K = kk[b, :, h].float().cpu().numpy()[None, None]
        V = vv[b, :, h].float().cpu().numpy()[None, None]
        oc = T.oracle_layer(wb, K, V, _pair_meta(m, h), n_cap)
        for name in ("k_codes", "v_codes", "k_scale", "v_scale", "k_zero", "v_zero", "recent_k", "recent_v"):
            ref = getattr(oc, name)
            if ref is None:
                continue
            buf = getattr(cache, name)
            got = T.layer_view(buf, 1, 0, (w.B, w.Hkv) + ref.shape[2:])[b, h].cpu().numpy()
            if ref.dtype == np.float16:
                got, ref = got.view(np.uint16), ref.view(np.uint16)
            np.testing.assert_array_equal(got, ref[0, 0], f"{name} (b={b}, h={h})")
        ref = pipeline.decode_layer(oc, q[b:b + 1, h * g:(h + 1) * g].float().cpu().numpy())
        e = T.assert_close(out[b:b + 1, h * g:(h + 1) * g], ref, f"workload {wid} b={b} h={h}")
        print(f"  pair (b={b}, h={h}): codes exact, max abs err {e:.2e}", flush=True)


def test_full_size_fp16_comparator():
    """The unquantized comparator at the headline shape (Qwen2.5-3B, 131072 tokens, 16 query / 2 kv
    heads) with the automatic split count the bench uses; every query head against the oracle."""
    w = synth.reduced(synth.WORKLOADS[2], L=1)
    N = w.N
    print(f"[full size] fp16 comparator: N={N} Hq={w.Hq} Hkv={w.Hkv}", flush=True)
    k16 = torch.stack([sg.keys(w, 0, h, 0, N) for h in range(w.Hkv)])[None].to(torch.float16)  # [1, Hkv, N, d]
    v16 = torch.stack([sg.values(w, 0, h, 0, N) for h in range(w.Hkv)])[None].to(torch.float16)
    q = torch.stack([torch.cat([sg.queries(w, 0, h, 0, N) for h in range(w.Hkv)])])
    import packed_cache_decode_block_amd as P
    out = P.bgtq_fp16_decode_attention(k16, v16, q, n_splits=0).cpu().numpy()
    ref = pipeline.fp16_decode(k16.cpu().numpy(), v16.cpu().numpy(), q.float().cpu().numpy())
    e = T.assert_close(out, ref, "fp16 comparator, full size")
    print(f"  max abs err {e:.2e}", flush=True)


def test_full_size_logquant_prefill():
    """LogQuant's filter over a 131072-token prompt in one call at the headline shape (Qwen2.5-3B:
    16 query / 2 kv heads, K3V3, W = 64): for kv head 0 the whole packed store equals the oracle's
    store of the leaving tokens in leaving order (bit-exact), the high-precision store holds the kept
    rows, and the decode over both matches the oracle."""
    from oracle import logquant as lq
    import packed_cache_decode_block_amd as P
    w = synth.reduced(synth.WORKLOADS[2], L=1)
    N, W, g = w.N, 64, w.g
    kept, left = lq.select(N, W)
    n_cap = (len(left) + 63) // 64 * 64
    print(f"[full size] log-based filter prefill: N={N} W={W}: {len(left)} packed + {len(kept)} fp16", flush=True)
    m = T.meta(w, 0)
    cache = P.PackedCache(L=1, B=1, Hq=w.Hq, Hkv=w.Hkv, n_cap=n_cap, budget_units=w.k_budget_units,
                          v_bits=w.v_bits, logquant_w=W)
    cache.set_metadata(0, m.bits, m.sigma, m.r)
    kk = torch.stack([sg.keys(w, 0, h, 0, N) for h in range(w.Hkv)], dim=1)[None]     # [1, N, Hkv, d]
    vv = torch.stack([sg.values(w, 0, h, 0, N) for h in range(w.Hkv)], dim=1)[None]
    q = torch.stack([torch.cat([sg.queries(w, 0, h, 0, N) for h in range(w.Hkv)])])
    cache.logquant_prefill(0, kk, vv)
    out = cache.decode_attention(0, q).cpu().numpy()
    torch.cuda.synchronize()
    assert cache.n_tokens[0, 0] == N and cache.n_hp[0, 0] == len(kept) and cache.hp_pos[0, 0, :len(kept)].tolist() == kept
    h = 0
    K = kk[0, :, h].float().cpu().numpy()
    V = vv[0, :, h].float().cpu().numpy()
    k16 = K[left].astype(np.float16).astype(np.float32)[None, None]
    v16 = V[left].astype(np.float16).astype(np.float32)[None, None]
    wb = synth.reduced(w, B=1, Hkv=1, Hq=g)
    oc = pipeline.build_layer(k16, v16, k_mode="gtq", v_mode="codebook", v_bits=w.v_bits, n_cap=n_cap,
                              meta=_pair_meta(m, h))
    for name in ("k_codes", "v_codes", "k_scale", "v_scale"):
        ref = getattr(oc, name)
        got = T.layer_view(getattr(cache, name), 1, 0, (1, w.Hkv) + ref.shape[2:])[0, h].cpu().numpy()
        if ref.dtype == np.float16:
            got, ref = got.view(np.uint16), ref.view(np.uint16)
        np.testing.assert_array_equal(got, ref[0, 0], f"{name} (h={h})")
    oc.recent_k = K[kept].astype(np.float16)[None, None]
    oc.recent_v = V[kept].astype(np.float16)[None, None]
    oc.n_recent_valid = len(kept)
    ref = pipeline.decode_layer(oc, q[:, h * g:(h + 1) * g].float().cpu().numpy())
    e = T.assert_close(out[:, h * g:(h + 1) * g], ref, "prefill full size")
    print(f"  kv head {h}: packed store exact, max abs err {e:.2e}", flush=True)
