"""CPU oracle for packed-cache decode attention over a Block-GTQ KV cache.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this package.  It shares
no code, table or constant generator with the HIP library; neither imports the other.

Plain, slow, obviously-correct NumPy: float64 for attention, and float32 emulated one IEEE
operation at a time (no fused multiply-add, sequential sums) where the method's integer
outputs (codes, scales) depend on floating-point decisions.

Sources (web pages on the method; cited by title and section):
  * "RoPE-Aware Bit Allocation for KV-Cache Quantization" — a review page (sections
    1 Key Terms, 2 Motivation, 3 Method & Key Results, Figures 1-2) and the paper's
    abstract page (Korean and English abstract).  Primary for Block-GTQ.
  * "Quantize What Counts: more for keys, less for values" — a technical summary
    (Results: K4V2 memory, group-size sensitivity).  Grounds the affine K4/V2 variant.
  * "LogQuant" — a technical summary (Method 2: high-precision recent window; Method 4:
    position-agnostic concatenation A·V = A_P·V_P).  Grounds the fp16 recent buffer.

Modules: codebook (Lloyd-Max tables), energy (calibration scores), allocate (greedy widths),
quantize (per-token codes and scales), layout (byte layout of the packed cache),
attention (dequantization, fp64 attention, split merge), pipeline (cache build + decode).

Parity status: every function is pinned by ``tests/test_oracle_*.py`` against closed forms,
textbook values, brute force or invariants.  What no page fixes (the exact energy formula,
the codebook, the packed layout) follows the readings listed in the design notes; whether
those readings match the authors' own code is unpinned, since that code is not available.
"""
