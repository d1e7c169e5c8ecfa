"""Value reconstruction error with and without the value rotation (test infrastructure).

The "Quantize What Counts" summary (Results, rotation integration) finds that rotating the values
alone brings marginal or negative results, while rotating the keys recovers most of the K4V4
accuracy at K4V2.  This script measures the value side on the synthetic heads with the oracle's
own steps: every value row quantized as stored (per-token TQ-MSE codebook, or one affine group of
128), with and without the randomized Hadamard rotation y = H (s * v) / 16 (fp32 fast transform),
dequantized exactly and rotated back in fp64, then
  relative MSE = sum (v_hat - v)^2 / sum v^2   and
  output error = |o_hat - o| / |o| for the decode output over exact keys (the value error alone),
over the synthetic value rows of the workloads, and over the same rows with two channels scaled by
10 (an outlier-channel stress case that the synthetic heads do not have).

    python -m oracle.report_value_rotation [--tokens 2048]
"""
from __future__ import annotations

import argparse
import sys

import numpy as np

from . import attention, quantize


def _signs(seed: int, d: int = 128) -> np.ndarray:
    return np.where(np.random.default_rng(seed).random(d) < 0.5, -1.0, 1.0)


def reconstruct(v: np.ndarray, mode: str, bits: int, signs=None) -> np.ndarray:
    """The rows as the cache stores and the decode reads them, float64, in the original space."""
    x = v if signs is None else quantize.hadamard_rotate_f32(v, signs)
    if mode == "codebook":
        codes, S = quantize.quantize_v(x, bits)
        y = attention.dequant_codebook(codes, S, bits)
    else:
        codes, sc, zr = quantize.quantize_affine(x, bits, 128)
        y = attention.dequant_affine(codes, sc, zr, 128)
    return y if signs is None else attention.unrotate_output(y, signs)


def measure(w, mode: str, bits: int, n_tokens: int, outliers: bool, heads=((0, 0), (1, 1))):
    import synth
    rel, out_err = {False: [], True: []}, {False: [], True: []}
    for layer, h in heads:
        v = synth.values(w, layer, h, 0, n_tokens).astype(np.float32)
        if outliers:
            v = v.copy()
            v[:, [7, 90]] *= 10.0
        K = synth.keys(w, layer, h, 0, n_tokens).astype(np.float64)
        q = synth.queries(w, layer, h, 0, n_tokens).astype(np.float64)
        o = attention.attend(q, K, v.astype(np.float64))
        for rot in (False, True):
            vh = reconstruct(v, mode, bits, _signs(100 + 7 * layer + h) if rot else None)
            rel[rot].append(np.sum((vh - v) ** 2) / np.sum(v.astype(np.float64) ** 2))
            oh = attention.attend(q, K, vh)
            out_err[rot].append(np.linalg.norm(oh - o) / np.linalg.norm(o))
    return {rot: (float(np.mean(rel[rot])), float(np.mean(out_err[rot]))) for rot in (False, True)}


def report(n_tokens: int = 2048, out=sys.stdout):
    import synth
    cases = [(2, "codebook", 3), (2, "codebook", 2), (2, "codebook", 4), (4, "affine", 2), (4, "affine", 4),
             (3, "codebook", 2)]
    print(f"Value reconstruction with and without the value rotation ({n_tokens} rows per head, "
          "two (layer, kv head) pairs per workload)", file=out)
    print("", file=out)
    print("| workload | values | rows | rel. MSE plain | rel. MSE rotated | output err plain | output err rotated |",
          file=out)
    print("|---|---|---|---:|---:|---:|---:|", file=out)
    res = {}
    for wid, mode, bits in cases:
        w = synth.WORKLOADS[wid]
        for outliers in (False, True):
            r = measure(w, mode, bits, n_tokens, outliers)
            res[(wid, mode, bits, outliers)] = r
            print(f"| {wid} | {mode} {bits}-bit | {'2 channels x10' if outliers else 'as generated'} | "
                  f"{r[False][0]:.5f} | {r[True][0]:.5f} | {r[False][1]:.5f} | {r[True][1]:.5f} |", file=out)
    return res


if __name__ == "__main__":
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--tokens", type=int, default=2048)
    a = ap.parse_args()
    report(a.tokens)
