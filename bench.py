#!/usr/bin/env python
"""Bench: packed-KV decode attention on one MI355X.

One step = decode attention for every layer of the workload (prep + split-K decode + combine per
layer, through the C ABI) with the packed cache, queries and outputs resident in HBM.  Prints one
JSON line: effective HBM GB/s over algorithmic bytes (codes, scales/zeros, fp16 recent tokens, q,
out), the decode kernel's roofline (HIP events recorded around every decode kernel's own
execution over a second pass of the timed steps, queued behind a GPU-side wait so that the host's
launch latency stays outside them), the unquantized fp16 comparator, and the CPU
oracle timed on a bounded sample.  The default run adds the same decode with every product on the
vector ALUs (vector_alu_decode) and the decode line of each other workload (per_workload).

Default workload: Qwen2.5-3B-shaped decode, 36 layers, 16 query / 2 KV heads, 131072 tokens,
batch 1, Block-GTQ K3 keys and 3-bit values, bf16 activations (synthetic inputs).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "packed-KV decode attention: effective HBM GB/s (% of peak) at 128K ctx"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def bytes_per_token_head(w) -> float:
    """Algorithmic bytes one packed (token, kv head) costs: codes + scales (+ zeros)."""
    if w.k_mode == "gtq":
        k = 2 * w.k_budget_units / 8 + 2
    else:
        k = w.k_bits * w.d / 8 + (w.d // w.k_group) * 4
    v = w.v_bits * w.d / 8 + (2 if w.v_mode == "codebook" else 4)
    return k + v


def layer_bytes(w, N: int) -> float:
    n_rec = min(N, w.n_recent)
    act = {"f32": 4, "f16": 2, "bf16": 2}[w.dtype]
    return (w.B * w.Hkv * ((N - n_rec) * bytes_per_token_head(w) + n_rec * 2 * w.d * 2)
            + w.B * w.Hq * w.d * (act + 4))


def decode_kernel_name(w, path: str = "auto") -> str:
    """The decode kernel a workload dispatches to: with at least four query heads per kv head the
    matrix-core kernels (plan-driven for Block-GTQ keys, the affine one for affine keys), everything
    else and the vector path the vector-ALU one."""
    if path == "auto" and w.Hq // w.Hkv >= 4:
        return "k_decode_gtq" if w.k_mode == "gtq" else "k_decode_mxa"
    return "k_decode"


def arithmetic(w, path: str = "auto"):
    """(dtype, description) of the arithmetic the workload's decode kernel runs."""
    if decode_kernel_name(w, path) != "k_decode":
        return "f16", (f"{w.dtype} activations in; q.k and P.V on the matrix cores with fp16 operands "
                       "(key centroids exact in fp16, the scaled query as fp16 high + low parts, softmax "
                       "weights rounded to fp16) accumulated in fp32; softmax and output in fp32")
    return "f32", (f"{w.dtype} activations in; q.k as fp32 FMAs on the vector ALUs; P.V as fp16 dot products "
                   "(fp16 centroids times softmax weights rounded to fp16) accumulated in fp32")


# Short names of the workloads in profile file names.
WORKLOAD_TAGS = {1: "1layer_4k", 2: "qwen2.5-3b_128k", 3: "llama3.1-8b_32k_b8", 4: "llama3.1-8b_64k_b2_affine",
                 5: "qwen2.5-3b_512k"}

# Source files each decode kernel is built from; a counter summary holds for the sha256 of these.
KERNEL_SOURCES = {
    "k_decode_gtq": ("bgtq_decode_gtq.hip", "bgtq_device.h"),
    "k_decode": ("bgtq_kernels.hip", "bgtq_device.h"),
    "k_decode_mxa": ("bgtq_kernels.hip", "bgtq_device.h"),
    "k_decode_fp16_mx": ("bgtq_kernels.hip", "bgtq_device.h"),
    "k_quant": ("bgtq_kernels.hip", "bgtq_device.h"),
    "k_quant_rows": ("bgtq_quant_rows.hip", "bgtq_device.h"),
}


def kernel_source_sha(kernel: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        h.update(open(os.path.join(ROOT, "packed_cache_decode_block_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def measured_traffic(wid: int, kernel: str = "k_decode_gtq"):
    """HBM bytes per launch of a kernel from the committed rocprofv3 counter summary of this
    workload (FETCH_SIZE and WRITE_SIZE scaled by a plain copy's readings), or None when there is
    none or the kernel source has changed since the counters were taken."""
    import re
    path = os.path.join(ROOT, "profiles", f"{kernel}_{WORKLOAD_TAGS.get(wid, '-')}_hbm_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    h = re.search(r"sha256\s+`([0-9a-f]{64})`", text)
    t = re.search(r"traffic_bytes_per_launch:\s*(\d+)", text)
    if not h or not t or h.group(1) != kernel_source_sha(kernel):
        return None
    return int(t.group(1))


def calibrate_layer(w, layer: int, device="cuda"):
    """Block-GTQ metadata of one layer through the library: calibration energy on the device, then
    the greedy widths (bits, sigma, inv_sigma as host arrays [Hkv, 64])."""
    import torch

    import packed_cache_decode_block_amd as P
    import synth
    td = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    cal = [synth.calibration(w, layer, h) for h in range(w.Hkv)]
    kc = torch.from_numpy(np.ascontiguousarray(np.stack([c[0] for c in cal], axis=1))).to(device).to(td)
    qc = torch.from_numpy(np.ascontiguousarray(
        np.concatenate([np.transpose(c[1], (1, 0, 2)) for c in cal], axis=1))).to(device).to(td)
    scores, sigma, inv_sigma = P.bgtq_block_energy(kc, qc)
    return P.bgtq_allocate(scores, w.k_budget_units), sigma, inv_sigma


def build_packed(w, device="cuda", uniform_keys=False, k_rotation=False):
    import torch

    import packed_cache_decode_block_amd as P
    import synth
    from synth import gpu as sg

    n_cap = (w.N - min(w.N, w.n_recent) + 63) // 64 * 64
    cache = P.PackedCache(L=w.L, B=w.B, Hq=w.Hq, Hkv=w.Hkv, n_cap=n_cap,
                          k_mode=P.K_BLOCKGTQ if w.k_mode == "gtq" else P.K_AFFINE,
                          budget_units=w.k_budget_units or 128, k_bits=w.k_bits or 4, k_group=w.k_group or 32,
                          v_mode=P.V_CODEBOOK if w.v_mode == "codebook" else P.V_AFFINE, v_bits=w.v_bits,
                          n_recent=w.n_recent, k_rotation=k_rotation, zero=False)
    td = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    qs = []
    for layer in range(w.L):
        if k_rotation:  # seeded +-1 signs of the key rotation, per (layer, kv head)
            rs = np.random.default_rng([w.wid, layer, 7]).random((w.Hkv, 128))
            cache.set_key_rotation(layer, np.where(rs < 0.5, -1.0, 1.0))
        if w.k_mode == "gtq":
            bits, sigma, inv_sigma = calibrate_layer(w, layer, device)
            if uniform_keys:  # uniform TQ-MSE keys: every block at the average width
                bits = np.full_like(bits, w.k_budget_units // 64)
            cache.set_metadata(layer, bits, sigma, inv_sigma)
        for b in range(w.B):
            k = torch.stack([sg.keys(w, layer, h, b, w.N, device) for h in range(w.Hkv)], dim=1)[None]
            v = torch.stack([sg.values(w, layer, h, b, w.N, device) for h in range(w.Hkv)], dim=1)[None]
            if b == 0:
                kk, vv = k, v
            else:
                kk, vv = torch.cat([kk, k]), torch.cat([vv, v])
        cache.quantize_append(layer, kk, vv)
        del kk, vv
        q = torch.stack([torch.cat([sg.queries(w, layer, h, b, w.N, device) for h in range(w.Hkv)])
                         for b in range(w.B)])
        qs.append(q)
    torch.cuda.synchronize()
    return cache, qs


def build_fp16(w, device="cuda"):
    """Unquantized comparator cache: the same synthetic rows in fp16, [B, Hkv, N, 128] per layer."""
    import torch

    from synth import gpu as sg
    ks, vs = [], []
    for layer in range(w.L):
        ks.append(torch.stack([torch.stack([sg.keys(w, layer, h, b, w.N, device) for h in range(w.Hkv)])
                               for b in range(w.B)]).to(torch.float16))
        vs.append(torch.stack([torch.stack([sg.values(w, layer, h, b, w.N, device) for h in range(w.Hkv)])
                               for b in range(w.B)]).to(torch.float16))
    torch.cuda.synchronize()
    return ks, vs


def timed(run_step, steps: int, warmup: int):
    import torch
    for _ in range(warmup):
        run_step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        run_step()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def queued(torch, run_step, steps: int, host_s: float):
    """Run the steps behind a GPU-side wait longer than the host needs to enqueue them, so that
    the GPU meets every launch already queued: events recorded around each kernel then time the
    kernel, not the host's launch latency.  host_s: the host's time for the steps (eager)."""
    if not hasattr(queued, "rate"):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)
        e0.record()
        torch.cuda._sleep(1_000_000)
        e1.record()
        torch.cuda.synchronize()
        queued.rate = 1_000_000 / max(e0.elapsed_time(e1) * 1e-3, 1e-6)  # sleep cycles per second
    torch.cuda.synchronize()
    torch.cuda._sleep(int(queued.rate * (1.5 * host_s + 0.005)))
    for _ in range(steps):
        run_step()
    torch.cuda.synchronize()


def time_decode(P, torch, cache, qs, outs, w, args, graph: bool = True):
    """Decode step over every layer: eager step time, the decode kernel's event-timed duration over
    a second pass of the steps, and the step replayed from a HIP graph (every layer's prep, decode
    and merge; no host launch overhead between them; eager if capture fails)."""
    ws = cache.workspace(args.n_splits)

    def step():
        for layer in range(w.L):
            cache.decode_attention(layer, qs[layer], outs[layer], n_splits=args.n_splits, ws=ws)

    sec_eager = timed(step, args.steps, args.warmup)       # eager launches, no tracing
    P.bgtq_profile_enable(w.L * args.steps)
    queued(torch, step, args.steps, sec_eager * args.steps)
    n_k, tot_ms, min_ms, max_ms = P.bgtq_profile_read(P.PROF_DECODE)
    P.bgtq_profile_enable(0)
    r = {"sec": sec_eager, "sec_eager": sec_eager, "graph_ok": False, "n_k": n_k,
         "kern_ms": tot_ms / max(n_k, 1), "min_ms": min_ms, "max_ms": max_ms, "step": step, "ws": ws}
    if graph and not args.eager:
        try:
            g = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                step()
            torch.cuda.current_stream().wait_stream(side)
            with torch.cuda.graph(g):
                step()
            r["sec"] = timed(g.replay, args.steps, args.warmup)
            r["graph_ok"] = True
            del g
        except Exception as e:  # capture unsupported: keep the eager number
            log(f"[bench] graph capture failed ({e}); reporting eager launches")
    return r


def time_fp16(P, torch, w, qs, outs, args, sec_packed):
    """The unquantized comparator: the same rows in fp16, decoded by the library's fp16 kernel."""
    ks, vs = build_fp16(w)
    ws16 = torch.empty(P.lib.bgtq_fp16_decode_workspace_bytes(w.N, w.B, w.Hq, w.Hkv, args.n_splits),
                       dtype=torch.uint8, device="cuda")

    def step16():
        for layer in range(w.L):
            P.bgtq_fp16_decode_attention(ks[layer], vs[layer], qs[layer], outs[layer], args.n_splits, ws16)

    sec16 = timed(step16, args.steps, args.warmup)
    P.bgtq_profile_enable(w.L * args.steps)
    queued(torch, step16, args.steps, sec16 * args.steps)
    n16, tot16, _, _ = P.bgtq_profile_read(P.PROF_FP16_DECODE)
    P.bgtq_profile_enable(0)
    del ks, vs, ws16
    b16 = w.B * w.Hkv * w.N * 512 + w.B * w.Hq * w.d * 6
    k16_ms = tot16 / max(n16, 1)
    mx = w.Hq // w.Hkv >= 4
    return {"ms_per_step": round(sec16 * 1e3, 4), "value": round(w.L * b16 / sec16 / 1e9, 2), "unit": "GB/s",
            "kernel_avg_us": round(k16_ms * 1e3, 3),
            "kernel_GB/s": round(b16 / (k16_ms * 1e-3) / 1e9, 1),
            "kernel_frac": round(b16 / (k16_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "kernel": "k_decode_fp16_mx" if mx else "k_decode_fp16",
            "traffic": measured_traffic(w.wid, "k_decode_fp16_mx") if mx else None,
            "speedup_packed_vs_fp16": round(sec16 / sec_packed, 3)}


def per_workload(wid, args, P, torch, synth):
    """One workload's decode at its own shape.  Every layer of a workload has the same shape, so
    enough layers are timed for a step to stream more than the 256 MB Infinity Cache (copies of the
    layer when the workload has fewer); the one-layer 4K workload (279 KB) is timed as it is."""
    w = synth.WORKLOADS[wid]
    lb = layer_bytes(w, w.N)
    if wid != 1:
        w = synth.reduced(w, L=max(1, int(np.ceil(320e6 / lb))))
    cache, qs = build_packed(w)
    outs = [torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda") for _ in range(w.L)]
    r = time_decode(P, torch, cache, qs, outs, w, args)
    del cache
    torch.cuda.empty_cache()
    kname = decode_kernel_name(w)
    ach = lb / (r["kern_ms"] * 1e-3) / 1e9
    e = {"workload": w.name, "layers_timed": w.L, "launch": "hipgraph" if r["graph_ok"] else "eager",
         "ms_per_step": round(r["sec"] * 1e3, 4), "GB/s": round(w.L * lb / r["sec"] / 1e9, 2),
         "tokens_heads_per_s": round(w.B * w.N * w.Hq * w.L / r["sec"], 1),
         "kernel": kname, "kernel_avg_us": round(r["kern_ms"] * 1e3, 3), "bytes_per_launch": lb,
         "kernel_GB/s": round(ach, 1), "frac": round(ach / PEAK_HBM_GBS, 4),
         "traffic": measured_traffic(wid, kname), "dtype": arithmetic(w)[0]}
    if not args.no_fp16:
        e["fp16_baseline"] = time_fp16(P, torch, w, qs, outs, args, r["sec"])
    torch.cuda.empty_cache()
    log(f"[bench] workload {wid}: {kname} {r['kern_ms'] * 1e3:.2f} us per layer ({ach:.0f} GB/s, "
        f"frac {ach / PEAK_HBM_GBS:.3f}), step {r['sec'] * 1e3:.3f} ms over {w.L} layers")
    return e


def cpu_baseline(w, budget_s: float = 12.0):
    """The oracle (numpy, fp64) decoding a bounded sample: layer 0, the first N_s tokens of every
    (batch, kv head) of the first sequence, all query heads; repeated until ~budget_s seconds."""
    import synth
    from oracle import pipeline
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing
        blas = 1
    Ns = min(w.N, 16384)
    ws = synth.reduced(w, B=1, L=1, N=Ns, n_recent=min(w.n_recent, Ns // 2))
    m = None
    if ws.k_mode == "gtq":
        cal = [synth.calibration(ws, 0, h) for h in range(ws.Hkv)]
        m = pipeline.calibrate([c[0] for c in cal], [c[1] for c in cal], ws.k_budget_units)
    K = np.stack([synth.keys(ws, 0, h, 0, Ns) for h in range(ws.Hkv)])[None]
    V = np.stack([synth.values(ws, 0, h, 0, Ns) for h in range(ws.Hkv)])[None]
    q = np.concatenate([synth.queries(ws, 0, h, 0, Ns) for h in range(ws.Hkv)])[None]
    oc = pipeline.build_layer(K, V, k_mode=ws.k_mode, v_mode=ws.v_mode, v_bits=ws.v_bits,
                              n_cap=(Ns + 63) // 64 * 64, meta=m, k_bits=ws.k_bits or 4, k_group=ws.k_group or 32,
                              n_recent=ws.n_recent)
    def run(seconds):
        reps, t0 = 0, time.perf_counter()
        while True:
            pipeline.decode_layer(oc, q)
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds or reps >= 1000:
                return reps, el
    reps, el = run(budget_s)
    gbs = reps * layer_bytes(ws, Ns) / el / 1e9
    one = None
    try:  # the same oracle with its BLAS pool held to one thread
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            r1, e1 = run(budget_s / 3)
        one = {"value": round(r1 * layer_bytes(ws, Ns) / e1 / 1e9, 6), "seconds": round(e1, 2), "reps": r1}
    except ImportError:
        pass
    return {"value": round(gbs, 6), "unit": "GB/s", "cores": len(os.sched_getaffinity(0)),
            "blas_threads": blas, "kind": "oracle", "seconds": round(el, 2), "one_thread": one,
            "sample": f"layer 0 of 1, batch 1 of {w.B}, {Ns} of {w.N} tokens per kv head"
                      f" ({ws.n_recent} in the fp16 ring), all {w.Hq} query heads, {reps} decode repetitions"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=2, help="1..5 (see synth.WORKLOADS); 2 = headline")
    ap.add_argument("--n-splits", type=int, default=0, help="0 = the library's choice")
    ap.add_argument("--no-fp16", action="store_true", help="skip the fp16 comparator")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--layers", type=int, default=0, help="override the layer count (0 = workload's)")
    ap.add_argument("--eager", action="store_true", help="time eager launches only (no HIP graph replay)")
    ap.add_argument("--no-step", action="store_true", help="skip the append-then-attend decode step timing")
    ap.add_argument("--no-logquant", action="store_true", help="skip the log-based filter append timing")
    ap.add_argument("--k-rotation", action="store_true",
                    help="affine keys stored under the randomized Hadamard rotation (affine-key workloads)")
    ap.add_argument("--uniform-keys", action="store_true",
                    help="Block-GTQ keys with every block at the average width (the uniform comparator)")
    ap.add_argument("--decode-path", choices=("auto", "vector"), default="auto",
                    help="auto: the library's kernels; vector: every product on the vector ALUs (k_decode)")
    ap.add_argument("--no-vector", action="store_true", help="skip the vector-ALU decode leg of the default run")
    ap.add_argument("--no-per-workload", action="store_true",
                    help="skip the other workloads' decode lines of the default run")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MB",
                    help="only run a plain device copy of MB megabytes 5 times (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the decode path runs on one GPU's "
              "share of the heads and context", file=sys.stderr)
        sys.exit(2)

    import torch

    import packed_cache_decode_block_amd as P
    import synth

    if args.copy_probe:
        n = args.copy_probe * (1 << 20) // 4
        src = torch.randn(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy probe: 5 copies of {args.copy_probe} MiB (read {args.copy_probe} MiB, write "
            f"{args.copy_probe} MiB each)")
        return

    w = synth.WORKLOADS[args.workload]
    copies = 0
    if args.layers:
        w = synth.reduced(w, L=args.layers)
    elif w.L * layer_bytes(w, w.N) < 320e6 and w.wid != 1:
        # cold cache: cycle enough copies of the layer that a step streams more than the 256 MB
        # Infinity Cache holds (the one-layer 524K workload: 4 copies of its 88 MB)
        w = synth.reduced(w, L=int(np.ceil(320e6 / layer_bytes(w, w.N))))
        copies = w.L
        log(f"[bench] {w.L} layer copies cycled so that a step exceeds the 256 MB Infinity Cache")
    log(f"[bench] workload {w.wid}: {w.name}")
    t0 = time.perf_counter()
    P.bgtq_profile_enable(4 * w.L)   # time the quantize-append launches of the cache build
    if args.k_rotation and w.k_mode != "affine":
        print("--k-rotation applies to affine-key workloads (4)", file=sys.stderr)
        sys.exit(2)
    cache, qs = build_packed(w, uniform_keys=args.uniform_keys, k_rotation=args.k_rotation)
    nq, totq, _, _ = P.bgtq_profile_read(P.PROF_QUANTIZE)
    P.bgtq_profile_enable(0)
    log(f"[bench] packed cache built in {time.perf_counter() - t0:.1f}s")
    outs = [torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda") for _ in range(w.L)]
    if args.decode_path == "vector":
        cache.decode_path = P.DECODE_VECTOR
    r = time_decode(P, torch, cache, qs, outs, w, args)
    sec, sec_eager, graph_ok, ws = r["sec"], r["sec_eager"], r["graph_ok"], r["ws"]
    n_k, kern_ms, min_ms, max_ms = r["n_k"], r["kern_ms"], r["min_ms"], r["max_ms"]
    lb = layer_bytes(w, w.N)
    value = w.L * lb / sec / 1e9
    achieved = lb / (kern_ms * 1e-3) / 1e9
    log(f"[bench] step {sec * 1e3:.3f} ms ({'graph' if graph_ok else 'eager'}; eager {sec_eager * 1e3:.3f} ms) "
        f"({w.L} layers), decode kernel avg {kern_ms * 1e3:.2f} us "
        f"(min {min_ms * 1e3:.2f}, max {max_ms * 1e3:.2f}, n={n_k}) -> {achieved:.0f} GB/s")

    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(sec * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": arithmetic(w, args.decode_path)[0],
        "arithmetic": arithmetic(w, args.decode_path)[1], "data": "synthetic",
        "config": {"workload": w.name, "layers": w.L, "batch": w.B, "context": w.N, "q_heads": w.Hq,
                   "kv_heads": w.Hkv, "head_dim": w.d, "k_format": "blockgtq" if w.k_mode == "gtq" else "affine",
                   "k_bits_per_dim": (w.k_budget_units / 64) if w.k_mode == "gtq" else w.k_bits,
                   "v_bits": w.v_bits, "n_recent_fp16": w.n_recent, "activations": w.dtype,
                   "key_widths": "uniform" if args.uniform_keys else "greedy", "key_rotation": args.k_rotation,
                   "n_splits": args.n_splits or "auto", "layer_copies_cycled": copies,
                   "decode_path": args.decode_path},
        "pct_peak_hbm": round(100 * value / PEAK_HBM_GBS, 2),
        "launch": "hipgraph" if graph_ok else "eager", "ms_per_step_eager": round(sec_eager * 1e3, 4),
        "tokens_heads_per_s": round(w.B * w.N * w.Hq * w.L / sec, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(w.wid, decode_kernel_name(w, args.decode_path)),
                     "kernel": decode_kernel_name(w, args.decode_path), "kernel_avg_us": round(kern_ms * 1e3, 3),
                     "bytes_per_launch": lb, "launches_timed": n_k},
    }
    if args.decode_path == "auto" and not args.no_vector and decode_kernel_name(w) != "k_decode":
        # The same cache and queries with every product on the vector ALUs (no matrix-core
        # instructions): the kernel the library takes below four query heads per kv head.
        cache.decode_path = P.DECODE_VECTOR
        rv = time_decode(P, torch, cache, qs, outs, w, args)
        cache.decode_path = P.DECODE_AUTO
        ws = cache.workspace(args.n_splits)
        av = lb / (rv["kern_ms"] * 1e-3) / 1e9
        result["vector_alu_decode"] = {
            "decode_path": "vector", "kernel": "k_decode", "kernel_avg_us": round(rv["kern_ms"] * 1e3, 3),
            "bytes_per_launch": lb, "kernel_GB/s": round(av, 1), "frac": round(av / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic(w.wid, "k_decode"), "launches_timed": rv["n_k"],
            "ms_per_step": round(rv["sec"] * 1e3, 4), "launch": "hipgraph" if rv["graph_ok"] else "eager",
            "GB/s": round(w.L * lb / rv["sec"] / 1e9, 2), "dtype": arithmetic(w, "vector")[0],
            "arithmetic": arithmetic(w, "vector")[1],
            "matrix_core_speedup": round(rv["kern_ms"] / kern_ms, 3)}
        log(f"[bench] vector-ALU decode: k_decode {rv['kern_ms'] * 1e3:.2f} us per layer ({av:.0f} GB/s), "
            f"step {rv['sec'] * 1e3:.3f} ms")
    if nq:
        # write path: every packed (token, kv head) reads its K and V rows and writes its record
        es = {"f32": 4, "f16": 2, "bf16": 2}[w.dtype]
        n_pk = w.N - min(w.N, w.n_recent)
        qbytes = w.B * w.Hkv * n_pk * (2 * w.d * es + bytes_per_token_head(w))
        q_ms = totq / nq
        # 16-bit rows with Block-GTQ keys and codebook values take the register-row kernel (one
        # launch, key and value workgroups interleaved), every other format the tile kernel
        rows_path = w.dtype != "f32" and w.k_mode == "gtq" and w.v_mode == "codebook"
        qk = "k_quant_rows" if rows_path else "k_quant"
        result["quantize_append"] = {"kernel": qk, "launches": nq, "kernel_avg_us": round(q_ms * 1e3, 2),
                                     "tokens_per_launch": w.B * w.Hkv * n_pk, "bytes_per_launch": qbytes,
                                     "GB/s": round(qbytes / (q_ms * 1e-3) / 1e9, 1)}
        log(f"[bench] quantize-append {q_ms * 1e3:.1f} us per layer -> {qbytes / (q_ms * 1e-3) / 1e9:.0f} GB/s")
    if not args.no_step:
        # One decode step per layer: append one token per sequence, then attend over the grown
        # context (bgtq_decode_step), replayed from a HIP graph like the decode-only step.  The
        # step re-appends position N - 1 (the lengths are set back by one before capture), so the
        # attended context is the same N tokens; every replay rewrites that slot.  (With an fp16
        # window the slot the step evicts from already holds the newest row: other bytes, the
        # same work.)  Eager launches set the lengths back before every call.
        gen = torch.Generator(device="cuda").manual_seed(11)
        td = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
        kn = [torch.randn((w.B, 1, w.Hkv, w.d), generator=gen, device="cuda").to(td) for _ in range(w.L)]
        vn = [torch.randn((w.B, 1, w.Hkv, w.d), generator=gen, device="cuda").to(td) for _ in range(w.L)]
        qd = [x.to(td) for x in qs]

        def step_append():
            for layer in range(w.L):
                cache.n_tokens[layer] -= 1
                cache.decode_step(layer, kn[layer], vn[layer], qd[layer], outs[layer], n_splits=args.n_splits, ws=ws)

        if graph_ok:
            gs = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gs):
                step_append()
            sec_s = timed(gs.replay, args.steps, args.warmup)
            del gs
        else:  # eager launches, like the decode-only figure it is compared with
            sec_s = timed(step_append, args.steps, args.warmup)
        assert (cache.n_tokens == w.N).all()
        result["decode_step"] = {
            "entry": "bgtq_decode_step", "tokens_appended_per_sequence": 1, "ms_per_step": round(sec_s * 1e3, 4),
            "launch": "hipgraph" if graph_ok else "eager",
            "us_per_layer": round(sec_s * 1e6 / w.L, 2),
            "append_us_per_layer": round((sec_s - sec) * 1e6 / w.L, 2)}
        log(f"[bench] decode step (append 1 token + attend) {sec_s * 1e3:.3f} ms, "
            f"{sec_s * 1e6 / w.L:.2f} us per layer ({(sec_s - sec) * 1e6 / w.L:.2f} us for the append)")
    if not args.no_logquant and w.k_mode == "gtq":
        # LogQuant's log-based filter on this workload's format and layer-0 calibration, W = 64 (a
        # 192-row fp16 store): (1) one-token appends (bgtq_logquant_append), 2048 per kv head, a
        # halving every 64 tokens; wall time per call includes the host plan; the leaving rows'
        # quantize is event-timed; (2) a whole prompt of the workload's context in one call
        # (bgtq_logquant_prefill), event-timed quantize and wall time.
        from synth import gpu as sg
        W_lq, n_lq = 64, 2048
        bits0, sig0, inv0 = calibrate_layer(w, 0)
        td = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
        lqc = P.PackedCache(L=1, B=1, Hq=w.Hq, Hkv=w.Hkv, n_cap=n_lq, budget_units=w.k_budget_units,
                            v_bits=w.v_bits, logquant_w=W_lq)
        lqc.set_metadata(0, bits0, sig0, inv0)
        rows = [torch.stack([f(w, 0, h, 0, n_lq) for h in range(w.Hkv)], dim=1)[None].to(td)
                for f in (sg.keys, sg.values)]
        for p in range(3 * W_lq):   # fill the store (no timing)
            lqc.logquant_append(0, rows[0][:, p:p + 1], rows[1][:, p:p + 1])
        views = [(rows[0][:, p:p + 1], rows[1][:, p:p + 1]) for p in range(3 * W_lq, n_lq)]
        torch.cuda.synchronize()
        P.bgtq_profile_enable(n_lq)
        t0 = time.perf_counter()
        for kv in views:
            lqc.logquant_append(0, kv[0], kv[1])
        torch.cuda.synchronize()
        t_lq = time.perf_counter() - t0
        nq_lq, tq_lq, _, _ = P.bgtq_profile_read(P.PROF_QUANTIZE)
        P.bgtq_profile_enable(0)
        n_calls = n_lq - 3 * W_lq
        result["logquant_append"] = {
            "entry": "bgtq_logquant_append", "W": W_lq, "store_rows": 3 * W_lq, "calls": n_calls,
            "metadata": "calibrated (layer 0 of the workload)",
            "halvings": nq_lq, "us_per_call": round(t_lq * 1e6 / n_calls, 2),
            "leaving_quantize_us": round(tq_lq * 1e3 / max(nq_lq, 1), 2),
            "packed_after": int(lqc.n_tokens[0, 0] - lqc.n_hp[0, 0]), "fp16_after": int(lqc.n_hp[0, 0])}
        log(f"[bench] log-based filter: {t_lq * 1e6 / n_calls:.1f} us per one-token append (host plan included), "
            f"{nq_lq} halvings, leaving-row quantize {tq_lq * 1e3 / max(nq_lq, 1):.1f} us each")
        del lqc, rows, views
        # the prompt of the workload's full context, one call
        N_p = w.N
        pc = P.PackedCache(L=1, B=w.B, Hq=w.Hq, Hkv=w.Hkv, n_cap=N_p, budget_units=w.k_budget_units,
                           v_bits=w.v_bits, logquant_w=W_lq)
        pc.set_metadata(0, bits0, sig0, inv0)
        kp = torch.stack([torch.stack([sg.keys(w, 0, h, b, N_p) for h in range(w.Hkv)], dim=1) for b in range(w.B)])
        vp = torch.stack([torch.stack([sg.values(w, 0, h, b, N_p) for h in range(w.Hkv)], dim=1) for b in range(w.B)])
        pc.logquant_prefill(0, kp, vp)  # warm-up (then the layer is reset and filled again)
        torch.cuda.synchronize()
        pc.n_tokens[:] = 0
        pc.n_hp[:] = 0
        P.bgtq_profile_enable(4)
        t0 = time.perf_counter()
        pc.logquant_prefill(0, kp, vp)
        torch.cuda.synchronize()
        t_pf = time.perf_counter() - t0
        npf, tpf, _, _ = P.bgtq_profile_read(P.PROF_QUANTIZE)
        P.bgtq_profile_enable(0)
        n_pk = int(pc.n_tokens[0, 0] - pc.n_hp[0, 0])
        result["logquant_prefill"] = {
            "entry": "bgtq_logquant_prefill", "W": W_lq, "prompt_tokens": N_p, "packed": n_pk,
            "fp16": int(pc.n_hp[0, 0]), "ms_per_call": round(t_pf * 1e3, 3),
            "quantize_us": round(tpf * 1e3 / max(npf, 1), 1),
            "tokens_per_s": round(w.B * N_p / t_pf, 1)}
        log(f"[bench] log-based filter prefill of {N_p} tokens: {t_pf * 1e3:.2f} ms per call "
            f"(gathered quantize {tpf * 1e3 / max(npf, 1):.1f} us)")
        del pc, kp, vp
    del ws
    if not args.no_fp16:
        del cache
        torch.cuda.empty_cache()
        result["fp16_baseline"] = time_fp16(P, torch, w, qs, outs, args, sec)
        log(f"[bench] fp16 comparator step {result['fp16_baseline']['ms_per_step']:.3f} ms, "
            f"speedup {result['fp16_baseline']['speedup_packed_vs_fp16']:.2f}x")
    else:
        del cache
    del qs, outs
    torch.cuda.empty_cache()
    if args.workload == 2 and not args.layers and not args.no_per_workload and args.decode_path == "auto":
        result["per_workload"] = {str(i): per_workload(i, args, P, torch, synth) for i in (1, 3, 4, 5)}
    if not args.no_cpu:
        log("[bench] timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
