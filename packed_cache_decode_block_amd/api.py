"""Thin wrappers over the C ABI: marshal torch tensors / numpy arrays into pointers and sizes."""
from __future__ import annotations

import ctypes as C

import numpy as np

from . import _lib
from ._lib import check, lib

_DT = None


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    m = {torch.float32: _lib.F32, torch.float16: _lib.F16, torch.bfloat16: _lib.BF16}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _stream(stream=None):
    torch = _torch()
    if stream is not None:
        return C.c_void_p(stream.cuda_stream)
    try:  # the raw handle of the current stream, without building a Stream object
        return C.c_void_p(torch._C._cuda_getCurrentRawStream(torch.cuda.current_device()))
    except AttributeError:
        return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return C.c_void_p(t.data_ptr()) if t is not None else None


def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensor must be on the GPU")
        if t is not None and not t.is_contiguous():
            raise ValueError("tensor must be contiguous")


def bgtq_version() -> str:
    return lib.bgtq_version().decode()


def bgtq_codebook(bits: int):
    """(centroids fp16 [2^bits], thresholds fp32 [2^bits - 1]) of the library's frozen table."""
    n = 1 << bits if 1 <= bits <= 8 else 1
    c = np.zeros(n, np.uint16)
    t = np.zeros(max(n - 1, 1), np.float32)
    check(lib.bgtq_codebook(bits, c.ctypes.data_as(C.POINTER(C.c_uint16)), t.ctypes.data_as(C.POINTER(C.c_float))))
    return c.view(np.float16), t[: n - 1]


def bgtq_allocate(scores, budget_units: int, b_min: int = 0, b_max: int = 8, rate=None) -> np.ndarray:
    """Greedy widths: scores [n_heads, n_blk] fp64 -> uint8 [n_heads, n_blk] (host).  rate: None
    ranks gains by 4^-b; else D(b) for b = 0..b_max (bgtq_allocate_rate)."""
    s = np.ascontiguousarray(scores, dtype=np.float64)
    if s.ndim == 1:
        s = s[None]
    out = np.zeros(s.shape, np.uint8)
    sp, op = s.ctypes.data_as(C.POINTER(C.c_double)), out.ctypes.data_as(C.POINTER(C.c_uint8))
    if rate is None:
        check(lib.bgtq_allocate(sp, s.shape[0], s.shape[1], budget_units, b_min, b_max, op))
    else:
        r = np.ascontiguousarray(rate, dtype=np.float64)
        if r.ndim != 1 or r.shape[0] < b_max + 1:
            raise ValueError("rate needs b_max + 1 entries")
        check(lib.bgtq_allocate_rate(sp, s.shape[0], s.shape[1], budget_units, b_min, b_max,
                                     r.ctypes.data_as(C.POINTER(C.c_double)), op))
    return out


class LogQuantPlanner:
    """Host bookkeeping of one sequence's high-precision store under LogQuant's log-based filter
    (bgtq_logquant_plan): which store rows leave for the low-bit store, how the store compacts,
    and where the new token's row goes."""

    def __init__(self, W: int, library=None):
        """library: a library exporting bgtq_logquant_plan (default: this package's)."""
        self.W = int(W)
        self.hp_pos = np.zeros(3 * self.W, np.int64)
        self.n_hp = 0
        self._lib = library if library is not None else lib

    def append(self, pos: int):
        """-> (evict_slots, moves [(src, dst)], new_slot) for the token at position pos."""
        n = C.c_int(self.n_hp)
        ev = np.zeros(self.W, np.int32)
        ms = np.zeros(self.W, np.int32)
        md = np.zeros(self.W, np.int32)
        nm, ns = C.c_int(0), C.c_int(0)
        p32 = C.POINTER(C.c_int32)
        k = check(self._lib.bgtq_logquant_plan(self.W, self.hp_pos.ctypes.data_as(C.POINTER(C.c_int64)), C.byref(n), pos,
                                         ev.ctypes.data_as(p32), ms.ctypes.data_as(p32), md.ctypes.data_as(p32),
                                         C.byref(nm), C.byref(ns)))
        self.n_hp = n.value
        return ev[:k].copy(), list(zip(ms[:nm.value].tolist(), md[:nm.value].tolist())), ns.value


def bgtq_block_energy(k_cal, q_cal, score_mode: int = _lib.SCORE_QK, stream=None):
    """k_cal [T, Hkv, 128], q_cal [T, Hq, 128] device tensors -> (scores fp64, sigma fp32, inv_sigma fp32)
    host arrays [Hkv, 64].  Synchronizes the stream."""
    torch = _torch()
    _require_cuda(k_cal, q_cal)
    T, Hkv, d = k_cal.shape
    g = q_cal.shape[1] // Hkv
    chunks = (T + _lib.ENERGY_CHUNK - 1) // _lib.ENERGY_CHUNK
    ws = torch.empty(chunks * Hkv * 64 * 2, dtype=torch.float64, device=k_cal.device)
    sc = np.zeros((Hkv, 64)); sg = np.zeros((Hkv, 64), np.float32); rs = np.zeros((Hkv, 64), np.float32)
    check(lib.bgtq_block_energy(_ptr(k_cal), _ptr(q_cal), _dtype_code(k_cal), T, Hkv, g, d, score_mode,
                                sc.ctypes.data_as(C.POINTER(C.c_double)), sg.ctypes.data_as(C.POINTER(C.c_float)),
                                rs.ctypes.data_as(C.POINTER(C.c_float)), _ptr(ws), ws.numel() * 8, _stream(stream)))
    return sc, sg, rs


class PackedCache:
    """Device buffers of a packed KV cache plus the descriptor the library reads.

    All buffers are torch tensors owned by this object (layer-major, see include/bgtq.h).
    """

    def __init__(self, *, L, B, Hq, Hkv, n_cap, k_mode=_lib.K_BLOCKGTQ, budget_units=128, k_bits=4, k_group=32,
                 v_mode=_lib.V_CODEBOOK, v_bits=2, n_recent=0, k_rotation=False, logquant_w=None, device="cuda",
                 zero=True, decode_path=_lib.DECODE_AUTO, v_rotation=False):
        """logquant_w: base window W of LogQuant's log-based filter; the recent buffers then hold the
        3W-row high-precision store (n_recent = 3W) and appends go through logquant_append.
        decode_path: DECODE_AUTO (the library's kernel choice) or DECODE_VECTOR (every product on the
        vector ALUs); also settable later through the attribute of the same name.
        v_rotation: values stored under a randomized Hadamard rotation (set_value_rotation)."""
        torch = _torch()
        if logquant_w is not None:
            n_recent = 3 * int(logquant_w)
        self.desc = _lib.CacheDesc()
        d = self.desc
        d.L, d.B, d.Hq, d.Hkv, d.d = L, B, Hq, Hkv, 128
        d.n_cap = n_cap
        d.k_mode, d.budget_units, d.k_bits, d.k_group = k_mode, budget_units, k_bits, k_group
        d.v_mode, d.v_bits, d.n_recent = v_mode, v_bits, n_recent
        d.decode_path = decode_path
        self.n_tokens = np.zeros((L, B), np.int64)
        d.n_tokens = self.n_tokens.ctypes.data_as(C.POINTER(C.c_int64))
        self.n_hp = self.hp_pos = None
        if logquant_w is not None:
            self.n_hp = np.zeros((L, B), np.int32)
            self.hp_pos = np.zeros((L, B, n_recent), np.int64)
            self._hp_ptr = [self.hp_pos[i].ctypes.data_as(C.POINTER(C.c_int64)) for i in range(L)]
            d.n_hp = self.n_hp.ctypes.data_as(C.POINTER(C.c_int32))
        alloc = torch.zeros if zero else torch.empty

        def buf(which, dtype):
            n = check(lib.bgtq_cache_bytes(C.byref(d), which))
            if n == 0:
                return None
            return alloc(n // torch.tensor([], dtype=dtype).element_size(), dtype=dtype, device=device)

        self.k_codes = buf(_lib.BUF_K_CODES, torch.uint8)
        self.v_codes = buf(_lib.BUF_V_CODES, torch.uint8)
        self.k_scale = buf(_lib.BUF_K_SCALE, torch.float16)
        self.k_zero = buf(_lib.BUF_K_ZERO, torch.float16)
        self.v_scale = buf(_lib.BUF_V_SCALE, torch.float16)
        self.v_zero = buf(_lib.BUF_V_ZERO, torch.float16)
        self.recent_k = buf(_lib.BUF_RECENT_K, torch.float16) if n_recent else None
        self.recent_v = buf(_lib.BUF_RECENT_V, torch.float16) if n_recent else None
        self.bits = torch.zeros((L, Hkv, 64), dtype=torch.uint8, device=device)
        self.sigma = torch.zeros((L, Hkv, 64), dtype=torch.float32, device=device)
        self.inv_sigma = torch.zeros((L, Hkv, 64), dtype=torch.float32, device=device)
        # sign bits of the randomized Hadamard key rotation (affine keys), [L, Hkv, 16]; see
        # set_key_rotation.  All signs +1 until set.
        self.k_rot = torch.zeros((L, Hkv, 16), dtype=torch.uint8, device=device) if k_rotation else None
        # sign bits of the value rotation, [L, Hkv, 16]; see set_value_rotation
        self.v_rot = torch.zeros((L, Hkv, 16), dtype=torch.uint8, device=device) if v_rotation else None
        # decode plan of each layer (Block-GTQ keys), written by bgtq_prepare_metadata in set_metadata
        self.plan = buf(_lib.BUF_PLAN, torch.uint8)
        for name in ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero", "recent_k", "recent_v",
                     "bits", "sigma", "inv_sigma", "k_rot", "plan", "v_rot"):
            setattr(d, name, _ptr(getattr(self, name)))
        self._ws = None
        self._lq_ws = None

    def set_key_rotation(self, layer: int, signs):
        """Signs s [Hkv, 128] (+1 / -1, host) of the key rotation of one layer: affine keys are
        stored as H (s * k) / 16 and the query is rotated to H (s * q) / 8 at decode."""
        torch = _torch()
        if self.k_rot is None:
            raise ValueError("the cache was created without k_rotation")
        sg = np.asarray(signs)
        if sg.shape != (self.desc.Hkv, 128) or not np.all(np.abs(sg) == 1):
            raise ValueError("signs must be [Hkv, 128] of +1 / -1")
        packed = np.packbits((sg < 0).astype(np.uint8), axis=1, bitorder="little")
        self.k_rot[layer].copy_(torch.from_numpy(packed))

    def set_value_rotation(self, layer: int, signs):
        """Signs s [Hkv, 128] (+1 / -1, host) of the value rotation of one layer: values are stored
        as H (s * v) / 16 and the decode output is rotated back to s * (H o') / 8."""
        torch = _torch()
        if self.v_rot is None:
            raise ValueError("the cache was created without v_rotation")
        sg = np.asarray(signs)
        if sg.shape != (self.desc.Hkv, 128) or not np.all(np.abs(sg) == 1):
            raise ValueError("signs must be [Hkv, 128] of +1 / -1")
        packed = np.packbits((sg < 0).astype(np.uint8), axis=1, bitorder="little")
        self.v_rot[layer].copy_(torch.from_numpy(packed))

    def set_metadata(self, layer: int, bits, sigma, inv_sigma):
        """Upload per-(kv head, block) widths and key scales of one layer (host arrays [Hkv, 64])."""
        torch = _torch()
        b = np.asarray(bits)
        d = self.desc
        if b.shape != (d.Hkv, 64) or b.min() < 0 or b.max() > 8:
            raise ValueError("bits must be [Hkv, 64] widths in 0..8")
        if d.k_mode == _lib.K_BLOCKGTQ and np.any(b.sum(axis=1) != d.budget_units):
            raise ValueError(f"the widths of every kv head must sum to budget_units ({d.budget_units})")
        self.bits[layer].copy_(torch.from_numpy(np.ascontiguousarray(bits, np.uint8)))
        self.sigma[layer].copy_(torch.from_numpy(np.ascontiguousarray(sigma, np.float32)))
        self.inv_sigma[layer].copy_(torch.from_numpy(np.ascontiguousarray(inv_sigma, np.float32)))
        if d.k_mode == _lib.K_BLOCKGTQ:
            check(lib.bgtq_prepare_metadata(C.byref(d), layer, _stream()))

    @staticmethod
    def _kv_strides(k, v):
        if not (k.is_cuda and v.is_cuda):
            raise ValueError("k and v must be on the GPU")
        if k.shape != v.shape or k.dtype != v.dtype or k.stride() != v.stride():
            raise ValueError("k and v must have the same shape, dtype and strides")
        if k.dim() != 4 or k.stride(-1) != 1:
            raise ValueError("k and v must be [B, n_new, Hkv, 128] with head_dim contiguous")
        return (C.c_int64 * 3)(k.stride(0), k.stride(1), k.stride(2))

    def quantize_append(self, layer: int, k, v, stream=None):
        """Append rows k, v [B, n_new, Hkv, 128] (any strides in B/token/head, dim contiguous)."""
        strides = self._kv_strides(k, v)
        check(lib.bgtq_quantize_append(C.byref(self.desc), layer, _ptr(k), _ptr(v), _dtype_code(k), k.shape[1],
                                       strides, _stream(stream)))

    def _lq_workspace(self, n_prompt: int, device):
        torch = _torch()
        n = check(lib.bgtq_logquant_workspace_bytes(C.byref(self.desc), n_prompt))
        if n == 0:
            return None, 0
        if self._lq_ws is None or self._lq_ws.numel() < n + 256:
            self._lq_ws = torch.empty(n + 256, dtype=torch.uint8, device=device)
        p = self._lq_ws.data_ptr()
        return C.c_void_p((p + 255) // 256 * 256), n

    def logquant_append(self, layer: int, k, v, stream=None):
        """Append one token per sequence, k, v [B, 1, Hkv, 128], under the log-based filter."""
        if self.n_hp is None:
            raise ValueError("the cache was built without logquant_w")
        strides = self._kv_strides(k, v)
        if tuple(k.shape) != (self.desc.B, 1, self.desc.Hkv, 128):
            raise ValueError(f"k and v must be [{self.desc.B}, 1, {self.desc.Hkv}, 128]: one token per sequence")
        ws, n = self._lq_workspace(0, k.device)
        check(lib.bgtq_logquant_append(C.byref(self.desc), layer, _ptr(k), _ptr(v), _dtype_code(k), strides,
                                       self._hp_ptr[layer], ws, n, _stream(stream)))

    def logquant_prefill(self, layer: int, k, v, stream=None):
        """Start a layer from a prompt, k, v [B, n_prompt, Hkv, 128], under the log-based filter, in
        one call: the filter's selection over the prompt, one gathered quantize of the tokens that
        leave the high-precision store, and the kept rows written to the store."""
        if self.n_hp is None:
            raise ValueError("the cache was built without logquant_w")
        strides = self._kv_strides(k, v)
        ws, n = self._lq_workspace(k.shape[1], k.device)
        check(lib.bgtq_logquant_prefill(C.byref(self.desc), layer, _ptr(k), _ptr(v), _dtype_code(k), k.shape[1],
                                        strides, self._hp_ptr[layer], ws, n, _stream(stream)))

    def decode_step(self, layer: int, k, v, q, out=None, n_splits: int = 0, ws=None, stream=None):
        """Append k, v [B, n_new, Hkv, 128], then attend q [B, Hq, 128] over the grown context -> fp32 out."""
        torch = _torch()
        strides = self._kv_strides(k, v)
        _require_cuda(q)
        if q.dtype != k.dtype:
            raise ValueError("q, k and v must share a dtype")
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        if ws is None:
            ws = self.workspace(n_splits, q.device)
        check(lib.bgtq_decode_step(C.byref(self.desc), layer, _ptr(k), _ptr(v), _ptr(q), _dtype_code(q), k.shape[1],
                                   strides, _ptr(out), _ptr(ws), ws.numel(), n_splits, _stream(stream)))
        return out

    @property
    def decode_path(self) -> int:
        return self.desc.decode_path

    @decode_path.setter
    def decode_path(self, path: int):
        self.desc.decode_path = int(path)

    def workspace_bytes(self, n_splits: int = 0) -> int:
        return check(lib.bgtq_decode_workspace_bytes(C.byref(self.desc), n_splits))

    def workspace(self, n_splits: int = 0, device="cuda"):
        torch = _torch()
        n = self.workspace_bytes(n_splits)
        if self._ws is None or self._ws.numel() < n:
            self._ws = torch.empty(n + 256, dtype=torch.uint8, device=device)
        return self._ws

    def decode_attention(self, layer: int, q, out=None, n_splits: int = 0, ws=None, stream=None):
        """q [B, Hq, 128] -> out fp32 [B, Hq, 128]."""
        torch = _torch()
        _require_cuda(q)
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        if ws is None:
            ws = self.workspace(n_splits, q.device)
        check(lib.bgtq_decode_attention(C.byref(self.desc), layer, _ptr(q), _dtype_code(q), _ptr(out), _ptr(ws),
                                        ws.numel(), n_splits, _stream(stream)))
        return out


    def decode_attention_noalloc(self, layer: int, q, out, n_splits: int = 0, stream=None):
        """As decode_attention, with the partials in the library's fixed per-GPU scratch (no workspace;
        out must be given, so the call allocates nothing)."""
        _require_cuda(q, out)
        check(lib.bgtq_decode_attention_noalloc(C.byref(self.desc), layer, _ptr(q), _dtype_code(q), _ptr(out),
                                                n_splits, _stream(stream)))
        return out


def bgtq_fp16_decode_attention(k16, v16, q, out=None, n_splits: int = 0, ws=None, stream=None):
    """Unquantized comparator: k16, v16 fp16 [B, Hkv, N, 128]; q [B, Hq, 128] -> fp32 [B, Hq, 128]."""
    torch = _torch()
    _require_cuda(k16, v16, q)
    B, Hkv, N, d = k16.shape
    Hq = q.shape[1]
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if ws is None:
        n = check(lib.bgtq_fp16_decode_workspace_bytes(N, B, Hq, Hkv, n_splits))
        ws = torch.empty(n, dtype=torch.uint8, device=q.device)
    check(lib.bgtq_fp16_decode_attention(_ptr(k16), _ptr(v16), N, B, Hq, Hkv, d, _ptr(q), _dtype_code(q), _ptr(out),
                                         _ptr(ws), ws.numel(), n_splits, _stream(stream)))
    return out


def bgtq_profile_enable(max_launches: int) -> None:
    """Bracket up to max_launches main-kernel launches with HIP events (0 disables)."""
    check(lib.bgtq_profile_enable(max_launches))


def bgtq_profile_read(kind: int):
    """(count, total_ms, min_ms, max_ms) of the recorded launches of one kind; clears them."""
    n = C.c_int(0)
    tot, mn, mx = C.c_double(0), C.c_double(0), C.c_double(0)
    check(lib.bgtq_profile_read(kind, C.byref(n), C.byref(tot), C.byref(mn), C.byref(mx)))
    return n.value, tot.value, mn.value, mx.value
