"""Per-layer RoPE-logit MAE of Block-GTQ widths against uniform widths (test infrastructure).

The abstract compares, per layer, the mean absolute error of RoPE query-key logits under K-only
quantization at 2 and 3 bits per dimension: Block-GTQ's greedy per-block widths against uniform
TQ-MSE at the same budget (it reports 32-80% lower MAE and every layer won).  This script makes
the same comparison on the synthetic heads of the Qwen2.5-3B-shaped workload (36 layers, 2 kv
heads, 8 query heads each), with the oracle's own steps: calibration energy -> greedy widths (or
the budget spread evenly), TQ-MSE key quantization, exact fp64 dequantization, and
MAE = mean |q . k_hat - q . k| over every (query, key) pair of the layer.

Inputs (synth): per (layer, kv head), N cached keys at positions 0..N-1 and the group's queries
at Q decode positions after them.  Nothing here runs on a GPU or reads the library.

    python -m oracle.report_logit_mae [--layers 36] [--tokens 1024] [--positions 4]
"""
from __future__ import annotations

import argparse
import sys

import numpy as np

from . import attention, pipeline, quantize


def layer_mae(w, layer: int, budget_units: int, n_tokens: int, n_pos: int):
    """(MAE with Block-GTQ widths, MAE with uniform widths) of one layer, over its kv heads."""
    import synth
    err = {"gtq": [], "uniform": []}
    for h in range(w.Hkv):
        kc, qc = synth.calibration(w, layer, h)
        meta = pipeline.calibrate([kc], [qc], budget_units)
        K = synth.keys(w, layer, h, 0, n_tokens)
        exact_k = K.astype(np.float64)
        Q = np.concatenate([synth.queries(w, layer, h, 0, n_tokens + p) for p in range(n_pos)]).astype(np.float64)
        exact = Q @ exact_k.T
        for name, bits in (("gtq", meta.bits[0]), ("uniform", np.full(64, budget_units // 64))):
            codes, S = quantize.quantize_k_gtq(K, meta.sigma[0], meta.r[0], bits)
            Kh = attention.dequant_k_gtq(codes, S, meta.sigma[0], bits)
            err[name].append(np.abs(Q @ Kh.T - exact))
    return float(np.mean(err["gtq"])), float(np.mean(err["uniform"]))


def report(layers: int = 36, n_tokens: int = 1024, n_pos: int = 4, budgets=(128, 192), out=sys.stdout):
    import synth
    w = synth.WORKLOADS[2]
    rows = {}
    for U in budgets:
        rows[U] = [layer_mae(w, layer, U, n_tokens, n_pos) for layer in range(min(layers, w.L))]
    print(f"Per-layer RoPE-logit MAE, Block-GTQ vs uniform widths, {w.name}: "
          f"{n_tokens} keys and {n_pos} query positions x {w.g} heads per kv head, all {w.Hkv} kv heads", file=out)
    print("", file=out)
    print("| budget | layers won | MAE reduction min | median | max | mean MAE Block-GTQ | mean MAE uniform |", file=out)
    print("|---|---:|---:|---:|---:|---:|---:|", file=out)
    summary = {}
    for U, r in rows.items():
        g = np.array([a for a, _ in r]); u = np.array([b for _, b in r])
        red = 1.0 - g / u
        summary[U] = dict(won=int(np.sum(g < u)), layers=len(r), red_min=float(red.min()),
                          red_med=float(np.median(red)), red_max=float(red.max()))
        print(f"| K{U // 64} ({U} units) | {summary[U]['won']}/{len(r)} | {100 * red.min():.1f}% | "
              f"{100 * np.median(red):.1f}% | {100 * red.max():.1f}% | {g.mean():.4f} | {u.mean():.4f} |", file=out)
    print("", file=out)
    print("| layer | " + " | ".join(f"K{U // 64} Block-GTQ | K{U // 64} uniform | reduction" for U in rows) + " |", file=out)
    print("|---:|" + "---:|---:|---:|" * len(rows), file=out)
    for layer in range(len(next(iter(rows.values())))):
        cells = []
        for U, r in rows.items():
            g, u = r[layer]
            cells.append(f"{g:.4f} | {u:.4f} | {100 * (1 - g / u):.1f}%")
        print(f"| {layer} | " + " | ".join(cells) + " |", file=out)
    return summary


if __name__ == "__main__":
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--layers", type=int, default=36)
    ap.add_argument("--tokens", type=int, default=1024)
    ap.add_argument("--positions", type=int, default=4)
    a = ap.parse_args()
    report(a.layers, a.tokens, a.positions)
