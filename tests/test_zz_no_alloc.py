"""The decode entry point that allocates nothing (bgtq_decode_attention_noalloc): its output against
bgtq_decode_attention's on the same cache and query, through the C ABI, on two calls in a row, the
second with a smaller input (fewer sequences, shorter context) so that partials a previous call
left in the library's scratch cannot leak into the result; plus the oracle bar and the size limit."""
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
from packed_cache_decode_block_amd import _lib  # noqa: E402


def _setup(wid, ov, N):
    w = synth.reduced(synth.WORKLOADS[wid], **ov)
    n_cap = ((N + 63) // 64 + 1) * 64
    m = T.meta(w, 0)
    K, V, q = T.inputs(w, 0, N)
    oc = T.oracle_layer(w, K, V, m, n_cap)
    cache = T.gpu_cache(w, n_cap)
    if m is not None:
        cache.set_metadata(0, m.bits, m.sigma, m.r)
    T.append_all(cache, 0, K, V, w.dtype)
    return w, cache, T.to_dev(q, w.dtype), pipeline.decode_layer(oc, q)


# (workload, overrides, N) of the first call, then of the smaller second call
PAIRS = {
    "gtq_g8": ((2, {"L": 1, "B": 3}, 5000 + 17), (2, {"L": 1, "B": 1}, 700 + 3)),
    "gtq_g4_b4": ((3, {"L": 1, "B": 4}, 2000 + 1), (3, {"L": 1, "B": 2}, 64)),
    "ring_k3v2": ((5, {}, 4000 + 9), (5, {}, 300)),
    "affine_k4v2": ((4, {"L": 1, "B": 2}, 2000 + 5), (4, {"L": 1, "B": 1}, 1000)),
}


@pytest.mark.parametrize("name", list(PAIRS))
def test_noalloc_matches_workspace_entry(name):
    for step, (wid, ov, N) in enumerate(PAIRS[name]):
        print(f"[noalloc {name} call {step}] workload {wid} {ov} N={N}", flush=True)
        w, cache, qd, ref = _setup(wid, ov, N)
        for ns in (0, 2):
            want = cache.decode_attention(0, qd, n_splits=ns)
            got = torch.full_like(want, float("nan"))
            cache.decode_attention_noalloc(0, qd, got, n_splits=ns)
            torch.cuda.synchronize()
            g, wv = got.cpu().numpy(), want.cpu().numpy()
            # the same kernels with the same split count: identical results
            np.testing.assert_array_equal(g, wv, f"{name} call {step} splits={ns}")
            e = T.assert_close(g, ref, f"{name} call {step} splits={ns} vs oracle")
            print(f"  splits={ns}: identical to the workspace entry; max abs err vs oracle {e:.2e}", flush=True)


def test_noalloc_rejects_partials_beyond_scratch():
    w, cache, qd, _ = _setup(2, {"L": 1, "B": 1}, 640)
    per_split = w.B * w.Hq * 132 * 4
    too_many = _lib.NOALLOC_SCRATCH_BYTES // per_split + 1
    out = torch.empty((w.B, w.Hq, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(P.BgtqError) as e:
        cache.decode_attention_noalloc(0, qd, out, n_splits=too_many)
    assert e.value.code == P.E_UNSUPPORTED and "scratch" in str(e.value)
    # a split count that fits still works afterwards
    cache.decode_attention_noalloc(0, qd, out, n_splits=too_many - 1)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
