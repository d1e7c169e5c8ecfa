"""Packed-cache decode attention over a Block-GTQ KV cache, for MI355X (gfx950).

Python face of the C ABI in include/bgtq.h (libbgtq.so, hand-written HIP kernels).  PyTorch is
used only for device memory and streams; every step of the path runs in the library.  Importing
fails if the library is not built; device calls fail if no GPU is present.
"""
from ._lib import (BgtqError, BF16, E_BUDGET, E_CAPACITY, E_HIP, E_INVALID, E_UNSUPPORTED, F16, F32,
                   K_AFFINE, K_BLOCKGTQ, LIB_PATH, SCORE_K, SCORE_QK, SYMBOLS, V_AFFINE, V_CODEBOOK, lib)
from ._lib import DECODE_AUTO, DECODE_VECTOR, PROF_DECODE, PROF_FP16_DECODE, PROF_QUANTIZE
from .api import (LogQuantPlanner, PackedCache, bgtq_allocate, bgtq_block_energy, bgtq_codebook, bgtq_fp16_decode_attention,
                  bgtq_profile_enable, bgtq_profile_read, bgtq_version)

__all__ = ["DECODE_AUTO", "DECODE_VECTOR", "PROF_DECODE", "PROF_FP16_DECODE", "PROF_QUANTIZE", "bgtq_profile_enable", "bgtq_profile_read",
           "LogQuantPlanner", "PackedCache", "bgtq_allocate", "bgtq_block_energy", "bgtq_codebook", "bgtq_fp16_decode_attention",
           "bgtq_version", "BgtqError", "lib", "LIB_PATH", "SYMBOLS", "F32", "F16", "BF16", "SCORE_QK", "SCORE_K",
           "K_BLOCKGTQ", "K_AFFINE", "V_CODEBOOK", "V_AFFINE", "E_INVALID", "E_UNSUPPORTED", "E_BUDGET",
           "E_CAPACITY", "E_HIP"]
