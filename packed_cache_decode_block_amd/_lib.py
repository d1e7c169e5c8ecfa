"""ctypes binding of libbgtq.so (the C ABI in include/bgtq.h).  Argument marshalling only."""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbgtq.so")

OK, E_INVALID, E_UNSUPPORTED, E_BUDGET, E_CAPACITY, E_HIP = 0, -1, -2, -3, -4, -5
F32, F16, BF16 = 0, 1, 2
SCORE_QK, SCORE_K = 0, 1
K_BLOCKGTQ, K_AFFINE = 0, 1
V_CODEBOOK, V_AFFINE = 0, 1
(BUF_K_CODES, BUF_V_CODES, BUF_K_SCALE, BUF_K_ZERO, BUF_V_SCALE, BUF_V_ZERO, BUF_RECENT_K,
 BUF_RECENT_V, BUF_META, BUF_PLAN) = range(10)
PLAN_BYTES = 512  # BGTQ_PLAN_BYTES
DECODE_AUTO, DECODE_VECTOR = 0, 1  # bgtq_cache.decode_path
MAX_BATCH = 64
ENERGY_CHUNK = 16  # BGTQ_ENERGY_CHUNK: calibration tokens per workgroup of bgtq_block_energy

SYMBOLS = ["bgtq_last_error", "bgtq_version", "bgtq_codebook", "bgtq_allocate", "bgtq_allocate_rate",
           "bgtq_logquant_plan", "bgtq_logquant_append", "bgtq_block_energy", "bgtq_cache_bytes", "bgtq_quantize_append", "bgtq_decode_workspace_bytes", "bgtq_decode_attention",
           "bgtq_decode_step", "bgtq_fp16_decode_workspace_bytes", "bgtq_fp16_decode_attention", "bgtq_profile_enable",
           "bgtq_profile_read", "bgtq_decode_attention_noalloc", "bgtq_prepare_metadata",
           "bgtq_logquant_workspace_bytes", "bgtq_logquant_prefill"]
NOALLOC_SCRATCH_BYTES = 4 << 20  # BGTQ_NOALLOC_SCRATCH_BYTES
PROF_DECODE, PROF_FP16_DECODE, PROF_QUANTIZE = 0, 1, 2


class BgtqError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"bgtq error {code}: {msg}")
        self.code = code


class CacheDesc(C.Structure):
    _fields_ = [("L", C.c_int32), ("B", C.c_int32), ("Hq", C.c_int32), ("Hkv", C.c_int32), ("d", C.c_int32),
                ("n_cap", C.c_int64),
                ("k_mode", C.c_int32), ("budget_units", C.c_int32), ("k_bits", C.c_int32), ("k_group", C.c_int32),
                ("v_mode", C.c_int32), ("v_bits", C.c_int32), ("n_recent", C.c_int32),
                ("k_codes", C.c_void_p), ("v_codes", C.c_void_p), ("k_scale", C.c_void_p), ("k_zero", C.c_void_p),
                ("v_scale", C.c_void_p), ("v_zero", C.c_void_p), ("recent_k", C.c_void_p), ("recent_v", C.c_void_p),
                ("bits", C.c_void_p), ("sigma", C.c_void_p), ("inv_sigma", C.c_void_p),
                ("n_tokens", C.POINTER(C.c_int64)), ("k_rot", C.c_void_p),
                ("n_hp", C.POINTER(C.c_int32)), ("plan", C.c_void_p), ("decode_path", C.c_int32),
                ("v_rot", C.c_void_p)]


def bind(path: str, optional=()):
    """Load a library exporting the C ABI of include/bgtq.h and declare its prototypes (names in
    `optional` may be absent, e.g. from the host-only test library)."""
    lib = C.CDLL(path)
    P, I, I64, SZ, D = C.c_void_p, C.c_int, C.c_int64, C.c_size_t, C.POINTER(C.c_double)
    F = C.POINTER(C.c_float)
    sig = {
        "bgtq_last_error": (C.c_char_p, []),
        "bgtq_version": (C.c_char_p, []),
        "bgtq_codebook": (I, [I, C.POINTER(C.c_uint16), F]),
        "bgtq_allocate": (I, [D, I, I, I, I, I, C.POINTER(C.c_uint8)]),
        "bgtq_allocate_rate": (I, [D, I, I, I, I, I, D, C.POINTER(C.c_uint8)]),
        "bgtq_block_energy": (I, [P, P, I, I64, I, I, I, I, D, F, F, P, SZ, P]),
        "bgtq_cache_bytes": (I64, [C.POINTER(CacheDesc), I]),
        "bgtq_quantize_append": (I, [C.POINTER(CacheDesc), I, P, P, I, I64, C.POINTER(C.c_int64), P]),
        "bgtq_decode_workspace_bytes": (I64, [C.POINTER(CacheDesc), I]),
        "bgtq_decode_attention": (I, [C.POINTER(CacheDesc), I, P, I, P, P, SZ, I, P]),
        "bgtq_decode_attention_noalloc": (I, [C.POINTER(CacheDesc), I, P, I, P, I, P]),
        "bgtq_prepare_metadata": (I, [C.POINTER(CacheDesc), I, P]),
        "bgtq_logquant_plan": (I, [I, C.POINTER(C.c_int64), C.POINTER(C.c_int), I64, C.POINTER(C.c_int32),
                                   C.POINTER(C.c_int32), C.POINTER(C.c_int32), C.POINTER(C.c_int), C.POINTER(C.c_int)]),
        "bgtq_logquant_append": (I, [C.POINTER(CacheDesc), I, P, P, I, C.POINTER(C.c_int64), C.POINTER(C.c_int64), P,
                                     SZ, P]),
        "bgtq_logquant_workspace_bytes": (I64, [C.POINTER(CacheDesc), I64]),
        "bgtq_logquant_prefill": (I, [C.POINTER(CacheDesc), I, P, P, I, I64, C.POINTER(C.c_int64), C.POINTER(C.c_int64),
                                      P, SZ, P]),
        "bgtq_decode_step": (I, [C.POINTER(CacheDesc), I, P, P, P, I, I64, C.POINTER(C.c_int64), P, P, SZ, I, P]),
        "bgtq_fp16_decode_workspace_bytes": (I64, [I64, I, I, I, I]),
        "bgtq_fp16_decode_attention": (I, [P, P, I64, I, I, I, I, P, I, P, P, SZ, I, P]),
        "bgtq_profile_enable": (I, [I]),
        "bgtq_profile_read": (I, [I, C.POINTER(C.c_int), D, D, D]),
    }
    for name, (res, args) in sig.items():
        if name in optional and not hasattr(lib, name):
            continue
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "(python packed_cache_decode_block_amd/build_lib.py)")
    return bind(LIB_PATH)


lib = _load()


def check(rc: int) -> int:
    if rc < 0:
        raise BgtqError(rc, lib.bgtq_last_error().decode())
    return rc
