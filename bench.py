"""Benchmark: Gated DSA layer decode tokens/s at a 131,072-token context on one MI355X.

One step = one dsa_layer_decode call on a batch of one sequence: indexer
scores over the whole key cache (32 heads x 128, bf16 keys with 5% planted
high-norm rows), exact top-2048, gated sparse attention with 64 query heads
over one shared 128-dim K/V head.  Inputs are seeded synthetic tensors that
are resident in HBM before timing starts; the step rotates over
`--rotate` distinct layer buffer sets so that every step streams its key
cache from HBM rather than from the 256 MiB Infinity Cache.

Prints one JSON line with the throughput, the roofline of the dominant
kernel (the indexer's stream of the key cache, timed live inside the timed
steps with HIP events attached to that kernel's dispatch on the stream it
runs on, see dsa_set_indexer_events) and the CPU oracle's throughput on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "indexer_decode_ctx131072_traffic.md")
# sources of the timed indexer kernel: a traffic figure measured on other
# sources is stale
KERNEL_SOURCES = ["long_context_sparse_dsa_amd/csrc/dsa_indexer.hip",
                  "long_context_sparse_dsa_amd/csrc/dsa_topk_tile.h",
                  "long_context_sparse_dsa_amd/csrc/dsa_device.h"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--workload", default="dec128k",
                    choices=["dec128k", "dec1m_b32_fp8", "prefill8k", "prefill8k_fp8",
                             "hybrid51", "tiny"],
                    help="dec128k (default, the headline metric); the others time the "
                         "same path on the batched 1M-context fp8 decode, on the 8K "
                         "prefill chunk (bf16, or fp8 query heads and keys on the fp8 "
                         "MFMA), on one 5:1 SWA/DSA hybrid decode step of a ragged "
                         "batch of 8, and on the tiny 4K-context decode parity shape")
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--rotate", type=int, default=None, help="distinct layer buffer sets")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall-time budget of the CPU oracle sample (0: skip)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="before timing, copy a buffer of this many MiB once (a reference "
                         "kernel of known traffic for hardware-counter runs)")
    a = ap.parse_args()
    dflt = {"dec128k": (200, 20, 16), "dec1m_b32_fp8": (20, 3, 1), "prefill8k": (5, 1, 1),
            "prefill8k_fp8": (5, 1, 1), "hybrid51": (50, 5, 1), "tiny": (200, 20, 1)}
    st, wu, rot = dflt[a.workload]
    a.steps = a.steps if a.steps is not None else st
    a.warmup = a.warmup if a.warmup is not None else wu
    a.rotate = a.rotate if a.rotate is not None else rot
    return a


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic():
    """Bytes per indexer launch from the committed counter summary, if it was
    taken on the current kernel sources (else None)."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    m = re.search(r"source_hash:\s*([0-9a-f]+)", text)
    b = re.search(r"bytes_per_launch:\s*([0-9]+)", text)
    if not m or not b or m.group(1) != kernel_source_hash():
        return None
    return int(b.group(1))


class HipEvents:
    """hipEvent_t handles through the HIP runtime torch already loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        ev = ctypes.c_void_p()
        if self.hip.hipEventCreate(ctypes.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return ev.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a),
                                        ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, e):
        self.hip.hipEventDestroy(ctypes.c_void_p(e))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU sharding of this path is described in DESIGN.md).", file=sys.stderr)
        sys.exit(2)
    import torch

    import long_context_sparse_dsa_amd as dsa
    from long_context_sparse_dsa_amd import workloads as W

    dsa.load()
    torch.cuda.set_device(0)
    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.workload in ("prefill8k", "prefill8k_fp8"):
        result = bench_prefill(args, torch, dsa, W)
    elif args.workload == "hybrid51":
        result = bench_hybrid(args, torch, dsa, W)
    else:
        result = bench_decode(args, torch, dsa, W)
    print(json.dumps(result), flush=True)


def bench_decode(args, torch, dsa, W):
    dev = "cuda"
    wl = {"dec128k": W.decode_128k, "dec1m_b32_fp8": W.decode_1m_b32_fp8,
          "tiny": W.tiny_decode}[args.workload]()
    L = max(wl.ctx_lens)
    sets = [W.make_inputs(wl, device=dev, seed_offset=i) for i in range(args.rotate)]
    ws = torch.empty(dsa.dsa_layer_decode_workspace_size(wl.B, L, wl.K, wl.Hq, wl.D),
                     dtype=torch.uint8, device=dev)
    outs = [torch.empty_like(s["q"]) for s in sets]
    torch.cuda.synchronize()

    # one marshalled C-ABI call per buffer set: the timed loop issues
    # dsa_layer_decode directly, without per-call Python argument checks
    calls = [dsa.prepare_layer_decode(s["q_idx"], s["w"], s["k_idx"], s["k_scale"], s["q"],
                                      s["k_cache"], s["v_cache"], s["gate"], wl.K, s["ctx_len"],
                                      s["cu_ctx"], L, outs[i], ws)
             for i, s in enumerate(sets)]
    hip = HipEvents()
    ev = [(hip.create(), hip.create()) for _ in range(args.steps)]
    set_events = dsa.load().dsa_set_indexer_events
    rot = [args.rotate]
    nxt = [0]   # next buffer set: the rotation continues across passes, so
    #             every step takes the least recently used set

    def call_next():
        calls[nxt[0] % rot[0]]()
        nxt[0] += 1

    def timed(n, warm, with_events=False, per_step=False):
        for _ in range(warm):
            call_next()
        if rot[0] > 1:
            flush_infinity_cache(torch)
        torch.cuda.synchronize()
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1 if per_step else 2)]
        marks[0].record()
        for i in range(n):
            if with_events:
                set_events(ctypes.c_void_p(ev[i][0]), ctypes.c_void_p(ev[i][1]))
            call_next()
            if per_step:
                marks[i + 1].record()
        marks[-1].record()
        torch.cuda.synchronize()
        set_events(None, None)
        if per_step:
            return [marks[i].elapsed_time(marks[i + 1]) for i in range(n)]
        return marks[0].elapsed_time(marks[1]) / n   # ms per step

    # ---- the timed region: K layer steps, inputs resident in HBM ----
    ms = timed(args.steps, args.warmup)
    tok_s = wl.B / (ms * 1e-3)
    # ---- the same K steps again with an event between consecutive steps
    # (per-step percentiles), then with the indexer kernel of each step
    # recording its own start / end events (attached to its dispatch); both
    # kept out of the headline figure, which the extra packets would slow ----
    per = sorted(timed(args.steps, 0, per_step=True))
    timed(args.steps, 0, with_events=True)
    idx_ms = [hip.elapsed_ms(a, b) for a, b in ev]
    ms_idx = sum(idx_ms) / len(idx_ms)
    for a, b in ev:
        hip.destroy(a)
        hip.destroy(b)
    # warm-cache figure (same buffer set every step), reported for context
    rot[0] = 1
    ms_warm = timed(args.steps, args.warmup)
    copy_gbs = measured_copy_bandwidth(torch)

    fp8 = wl.key_dtype == "fp8"
    key_bytes = sum(wl.ctx_lens) * (wl.d_I + 4 if fp8 else 2 * wl.d_I)   # keys (+ fp8 scales)
    idx_bytes = key_bytes + wl.B * (wl.H_I * wl.d_I * 2 + wl.H_I * 2)   # + query heads, weights
    achieved = idx_bytes / (ms_idx * 1e-3) / 1e9
    layer_bytes = key_bytes + wl.B * (wl.K * 2 * wl.D * 2 + (wl.H_I * wl.d_I + wl.H_I) * 2 +
                                      3 * wl.Hq * wl.D * 2)
    result = {
        "metric": "DSA layer decode tokens/s @128K ctx (indexer HBM GB/s, % roofline)",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.B, "ctx": L, "indexer": f"{wl.H_I}x{wl.d_I}",
                   "topk": wl.K, "q_heads": wl.Hq, "kv_heads": 1, "head_dim": wl.D,
                   "key_cache": wl.key_dtype, "planted_frac": wl.plant_frac,
                   "rotated_buffer_sets": args.rotate},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": read_traffic() if args.workload == "dec128k" else None,
                     "kernel": "index_decode_kernel (key-cache stream + Top-K tile reports)",
                     "kernel_us": round(ms_idx * 1e3, 3),
                     "algorithmic_bytes_per_launch": idx_bytes},
        "layer_roofline": {"algorithmic_bytes_per_step": layer_bytes,
                           "frac_of_hbm_peak": round(layer_bytes / (ms * 1e-3) / 1e9 /
                                                     HBM_PEAK_GBS, 4)},
        "step_ms_percentiles": percentiles(per),
        "measured_copy_gbs": round(copy_gbs, 1),
        "indexer_frac_of_measured_copy": round(achieved / copy_gbs, 4),
        "warm_cache": {"ms_per_step": round(ms_warm, 5),
                       "tokens_per_s": round(wl.B / (ms_warm * 1e-3), 1)},
    }
    if args.workload == "dec1m_b32_fp8":
        result["metric"] = "DSA layer decode tokens/s (batched 1M-context fp8 decode)"
    elif args.workload == "tiny":
        result["metric"] = "DSA layer decode tokens/s (4K-context parity shape)"
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(sets[0], wl, args.cpu_seconds)
    return result


def bench_hybrid(args, torch, dsa, W):
    """One decode step of the 5:1 hybrid: five sliding-window (128) attention
    layers, ungated, each with its own K/V cache, then one Gated DSA layer;
    ragged batch of 8 sequences."""
    dev = "cuda"
    wl = W.hybrid_5to1()
    nswa, window = wl.extra["swa_layers"], wl.extra["window"]
    L = max(wl.ctx_lens)
    ntot = sum(wl.ctx_lens)
    s = W.make_inputs(wl, device=dev)
    swa = []
    for i in range(nswa):
        swa.append({"q": W.randn_bf16((wl.B, wl.Hq, wl.D), wl.seed, f"swa{i}_q", dev),
                    "k": W.randn_bf16((ntot, wl.D), wl.seed, f"swa{i}_k", dev),
                    "v": W.randn_bf16((ntot, wl.D), wl.seed, f"swa{i}_v", dev),
                    "out": torch.empty(wl.B, wl.Hq, wl.D, dtype=torch.bfloat16, device=dev)})
    # the five window layers in one launch (the fused step), and the same
    # layers issued one dsa_sparse_attn call each (timed beside it)
    swa_fused = dsa.prepare_swa_decode_layers([x["q"] for x in swa], [x["k"] for x in swa],
                                              [x["v"] for x in swa], s["ctx_len"], s["cu_ctx"],
                                              L, [x["out"] for x in swa], window)
    swa_calls = [dsa.prepare_sparse_attn(x["q"], x["k"], x["v"], None, s["ctx_len"], s["cu_ctx"],
                                         L, x["out"], window=window) for x in swa]
    ws = torch.empty(dsa.dsa_layer_decode_workspace_size(wl.B, L, wl.K, wl.Hq, wl.D),
                     dtype=torch.uint8, device=dev)
    out = torch.empty_like(s["q"])
    dsa_call = dsa.prepare_layer_decode(s["q_idx"], s["w"], s["k_idx"], s["k_scale"], s["q"],
                                        s["k_cache"], s["v_cache"], s["gate"], wl.K, s["ctx_len"],
                                        s["cu_ctx"], L, out, ws)
    hip = HipEvents()
    ev = [(hip.create(), hip.create()) for _ in range(args.steps)]
    set_events = dsa.load().dsa_set_indexer_events

    def step():
        swa_fused()
        dsa_call()

    def step_per_layer():
        for c in swa_calls:
            c()
        dsa_call()

    def timed(n, warm, with_events, fn=step):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            if with_events:
                set_events(ctypes.c_void_p(ev[i][0]), ctypes.c_void_p(ev[i][1]))
            fn()
        e1.record()
        torch.cuda.synchronize()
        set_events(None, None)
        return e0.elapsed_time(e1) / n

    ms = timed(args.steps, args.warmup, False)
    ms_per_layer = timed(args.steps, args.warmup, False, step_per_layer)
    timed(args.steps, 0, True)
    ms_idx = sum(hip.elapsed_ms(a, b) for a, b in ev) / len(ev)
    for a, b in ev:
        hip.destroy(a)
        hip.destroy(b)
    idx_bytes = ntot * 2 * wl.d_I + wl.B * (wl.H_I * wl.d_I * 2 + wl.H_I * 2)
    dsa_bytes = idx_bytes + wl.B * (wl.K * 2 * wl.D * 2 + 3 * wl.Hq * wl.D * 2)
    swa_bytes = nswa * wl.B * (window * 2 * wl.D * 2 + 2 * wl.Hq * wl.D * 2)
    achieved = idx_bytes / (ms_idx * 1e-3) / 1e9
    result = {
        "metric": "5:1 SWA/DSA hybrid decode step tokens/s (ragged batch of 8)",
        "value": round(wl.B / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.B, "ctx_lens": wl.ctx_lens,
                   "swa_layers": nswa, "window": window, "dsa_layers": 1,
                   "indexer": f"{wl.H_I}x{wl.d_I}", "topk": wl.K, "q_heads": wl.Hq,
                   "head_dim": wl.D},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "index_decode_kernel (DSA layer)",
                     "kernel_us": round(ms_idx * 1e3, 3),
                     "algorithmic_bytes_per_launch": idx_bytes},
        "layer_roofline": {"algorithmic_bytes_per_step": dsa_bytes + swa_bytes,
                           "frac_of_hbm_peak": round((dsa_bytes + swa_bytes) / (ms * 1e-3) /
                                                     1e9 / HBM_PEAK_GBS, 4)},
        "window_layers_one_call_each": {"ms_per_step": round(ms_per_layer, 5),
                                        "tokens_per_s": round(wl.B / (ms_per_layer * 1e-3), 1)},
    }
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline_hybrid(s, swa, wl, args.cpu_seconds)
    return result


def bench_prefill(args, torch, dsa, W):
    """The 8K prefill chunk: tokens/s of dsa_layer_prefill, and the MFMA
    roofline of its indexer (timed with HIP events around back-to-back
    dsa_index_scores launches on the same stream)."""
    fp8 = args.workload == "prefill8k_fp8"
    wl = W.prefill_8k_fp8() if fp8 else W.prefill_8k()
    s = W.make_inputs(wl, device="cuda")
    L = wl.ctx_lens[0]
    ws = torch.empty(dsa.dsa_layer_prefill_workspace_size(wl.B, wl.T, L, wl.K, wl.Hq, wl.D),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(s["q"])

    def layer():
        dsa.dsa_layer_prefill(s["q_idx"], s["w"], s["k_idx"], s["k_scale"], s["q"], s["k_cache"],
                              s["v_cache"], s["gate"], wl.K, s["cu_q"], s["ctx_len"], s["cu_ctx"],
                              max_q=wl.T, max_ctx=L, out=out, ws=ws, q_scale=s["q_scale"])

    def timed(fn, n, warm):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    ms = timed(layer, args.steps, args.warmup)
    del ws
    torch.cuda.empty_cache()
    scores = torch.empty(wl.T, L, dtype=torch.float32, device="cuda")

    def indexer():
        dsa.dsa_index_scores(s["q_idx"], s["w"], s["k_idx"], s["k_scale"], s["ctx_len"],
                             s["cu_ctx"], cu_q=s["cu_q"], max_q=wl.T, max_ctx=L, scores=scores,
                             q_scale=s["q_scale"])

    ms_idx = timed(indexer, args.steps, args.warmup)
    p0 = L - wl.T
    visible = sum(p0 + i + 1 for i in range(wl.T))
    flops = visible * 2 * wl.H_I * wl.d_I
    achieved = flops / (ms_idx * 1e-3) / 1e12
    peak = 5000.0 if fp8 else 2500.0   # dense fp8 / bf16 MFMA, published
    result = {
        "metric": "DSA layer prefill tokens/s (8K chunk at 131K context; indexer MFMA TFLOP/s)",
        "value": round(wl.T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "queries": wl.T, "ctx": L,
                   "indexer": f"{wl.H_I}x{wl.d_I}", "topk": wl.K, "q_heads": wl.Hq,
                   "head_dim": wl.D, "indexer_queries": wl.q_dtype, "indexer_keys": wl.key_dtype},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None,
                     "kernel": "index_prefill_kernel", "kernel_us": round(ms_idx * 1e3, 1),
                     "algorithmic_flops_per_launch": flops},
    }
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline_prefill(s, wl, args.cpu_seconds)
    return result


_FLUSH = {}


def flush_infinity_cache(torch, mib=512):
    """Read a buffer twice the 256 MiB Infinity Cache, so that no layer
    buffer stays cached from set-up or warm-up.  The buffer is written once,
    on the first call; later calls only read it, so the cache is left
    holding clean lines and the timed steps do not pay for writing a
    flush's dirty lines back to HBM."""
    buf = _FLUSH.get(mib)
    if buf is None:
        buf = torch.ones(mib << 20, dtype=torch.uint8, device="cuda")
        _FLUSH[mib] = buf
        torch.cuda.synchronize()
    buf.view(torch.int64).amax()


def measured_copy_bandwidth(torch, mib=2048, reps=5):
    """Achievable HBM bandwidth on this GPU: best device-to-device copy of
    `mib` MiB (bytes read + bytes written per second), in GB/s."""
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    best = None
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1)
        best = t if best is None else min(best, t)
    del src, dst
    return 2 * n / (best * 1e-3) / 1e9


def percentiles(ms_list):
    import numpy as np
    a = np.asarray(ms_list)
    return {"p10": round(float(np.percentile(a, 10)), 5),
            "p50": round(float(np.percentile(a, 50)), 5),
            "p90": round(float(np.percentile(a, 90)), 5)}


def host_cores():
    n_aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None
    return {"nproc": n_aff, "cpu_count": os.cpu_count()}


def _host(s):
    return {k: (v.cpu() if hasattr(v, "cpu") else v) for k, v in s.items()}


def cpu_baseline(s, wl, budget):
    """The fp64 oracle, untuned, on host cores: whole decode steps of the
    first sequence of the batch, repeated for about `budget` seconds."""
    import numpy as np
    import oracle
    c = _host(s)
    L = wl.ctx_lens[0]
    one = {"q_idx": c["q_idx"][:1], "w": c["w"][:1], "k_idx": c["k_idx"][:L],
           "k_scale": None if c["k_scale"] is None else c["k_scale"][:L], "q": c["q"][:1],
           "k_cache": c["k_cache"][:L], "v_cache": c["v_cache"][:L], "gate": c["gate"][:1]}
    n = oracle.default_threads()

    def run(threads, secs):
        t0 = time.perf_counter()
        runs = 0
        while True:
            oracle.layer(one["q_idx"], one["w"], one["k_idx"], one["k_scale"], one["q"],
                         one["k_cache"], one["v_cache"], one["gate"], wl.K,
                         np.array([L], dtype=np.int32), nthreads=threads)
            runs += 1
            el = time.perf_counter() - t0
            if el >= secs or runs >= 100000:
                return runs, el

    runs, el = run(n, budget)
    runs1, el1 = run(1, budget / 4)
    return {"value": round(runs / el, 3), "unit": "tokens/s", "cores": n, "kind": "oracle",
            "value_1thread": round(runs1 / el1, 3), "host": host_cores(),
            "sample": f"{runs} whole decode-layer steps of one sequence (ctx {L}) in {el:.1f} s, "
                      f"fp64, {n} threads; {runs1} steps in {el1:.1f} s on 1 thread"}


def cpu_baseline_prefill(s, wl, budget):
    """The oracle on the last queries of the chunk (the costliest), for about
    `budget` seconds; tokens/s over the queries it finished."""
    import numpy as np
    import oracle
    c = _host(s)
    L = wl.ctx_lens[0]
    n = oracle.default_threads()
    t0 = time.perf_counter()
    done = 0
    while True:
        i = wl.T - 1 - done
        ctx = np.array([L - wl.T + i + 1], dtype=np.int32)
        if c.get("q_scale") is None:
            oracle.layer(c["q_idx"][i:i + 1], c["w"][i:i + 1], c["k_idx"], c["k_scale"],
                         c["q"][i:i + 1], c["k_cache"], c["v_cache"], c["gate"][i:i + 1], wl.K,
                         ctx, nthreads=n)
        else:   # fp8 query heads: the same three steps, composed
            sc = oracle.index_scores(c["q_idx"][i:i + 1], c["w"][i:i + 1], c["k_idx"],
                                     c["k_scale"], ctx_len=ctx, q_scale=c["q_scale"][i:i + 1],
                                     nthreads=n)
            sel = oracle.topk(sc, wl.K, ctx, nthreads=n)
            oracle.sparse_attn(c["q"][i:i + 1], c["k_cache"], c["v_cache"], idx=sel,
                               gate=c["gate"][i:i + 1], ctx_len=ctx, nthreads=n)
        done += 1
        el = time.perf_counter() - t0
        if el >= budget or done >= wl.T:
            break
    return {"value": round(done / el, 3), "unit": "tokens/s", "cores": n, "kind": "oracle",
            "sample": f"the last {done} queries of the chunk, one decode-shaped oracle call each "
                      f"(context up to {L}) in {el:.1f} s, fp64, {n} threads"}


def cpu_baseline_hybrid(s, swa, wl, budget):
    """The oracle on whole hybrid steps (five windowed attention layers and
    one DSA layer) of the batch's shortest sequence, for about `budget` s."""
    import numpy as np
    import oracle
    c = _host(s)
    b = int(np.argmin(wl.ctx_lens))
    L = wl.ctx_lens[b]
    r0 = int(sum(wl.ctx_lens[:b]))
    sw = [{k: v[b:b + 1].cpu() if k in ("q", "out") else v[r0:r0 + L].cpu()
           for k, v in x.items()} for x in swa]
    ctx = np.array([L], dtype=np.int32)
    n = oracle.default_threads()
    t0 = time.perf_counter()
    runs = 0
    while True:
        for x in sw:
            oracle.sparse_attn(x["q"], x["k"], x["v"], window=wl.extra["window"], ctx_len=ctx,
                               nthreads=n)
        oracle.layer(c["q_idx"][b:b + 1], c["w"][b:b + 1], c["k_idx"][r0:r0 + L], None,
                     c["q"][b:b + 1], c["k_cache"][r0:r0 + L], c["v_cache"][r0:r0 + L],
                     c["gate"][b:b + 1], wl.K, ctx, nthreads=n)
        runs += 1
        el = time.perf_counter() - t0
        if el >= budget or runs >= 100000:
            break
    return {"value": round(runs / el, 3), "unit": "tokens/s", "cores": n, "kind": "oracle",
            "sample": f"{runs} whole hybrid steps (5 SWA + 1 DSA layers) of one sequence "
                      f"(ctx {L}) in {el:.1f} s, fp64, {n} threads"}


if __name__ == "__main__":
    main()
