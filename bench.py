#!/usr/bin/env python3
"""Decode benchmark: a Llama-7B-shaped W4A16 layer stack on one MI355X.

One step = one decode pass of M tokens through 32 distinct layers, each with the
seven projections Wq, Wk, Wv, Wo (4096x4096), gate, up (11008x4096) and down
(4096x11008), quantized symmetric INT4 with 128-weight groups (scale = absmax/7),
every product a fused-dequant GEMV in the HIP library. Weights are drawn on the
device (seeded N(0, 0.02)) and quantized with the library's quantize_pack; the
whole step is captured once in a HIP graph and replayed.

Prints one JSON line: HBM throughput of the step (algorithmic bytes / time),
decode tokens/s, the dominant kernel's roofline (timed live with HIP events on
its own stream) and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A16 decode GEMV achieved HBM TB/s (% of peak); 7B-layer decode tok/s"
HBM_PEAK_GBS = 8000.0
LLAMA7B = [("wq", 4096, 4096), ("wk", 4096, 4096), ("wv", 4096, 4096), ("wo", 4096, 4096),
           ("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008)]
SCHEME = "sym4_g128"


def matrix_bytes(N: int, K: int, M: int) -> int:
    """Algorithmic HBM bytes of one sym4_g128 GEMV: codes + fp32 scales + x in + y out."""
    return N * K // 2 + N * (K // 128) * 4 + M * K * 2 + M * N * 4


def group_bytes(shapes, M: int) -> int:
    """Algorithmic bytes of one launch serving several matrices that share x (x read once)."""
    K = shapes[0][1]
    return sum(matrix_bytes(N, K, M) for N, K in shapes) - (len(shapes) - 1) * M * K * 2


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--M", type=int, default=1, help="decode tokens per step (1..16)")
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="CPU oracle time budget")
    ap.add_argument("--dominant-only", action="store_true",
                    help="only replay the dominant kernel (for counter collection)")
    return ap.parse_args()


def cpu_baseline(layer, xs_host, M, budget_s):
    """The oracle as it stands, on layer 0's matrices (host copies), until the budget."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    done_bytes, done, t0 = 0, [], time.perf_counter()
    for name, N, K in LLAMA7B:
        q = layer[name]
        codes = q.codes.cpu().numpy()
        scale = q.scale.cpu().numpy()
        ts = time.perf_counter()
        oracle.gemv_reference(codes, scale, None, SCHEME, xs_host[K])
        done_bytes += matrix_bytes(N, K, M)
        done.append(name)
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    layer_frac = done_bytes / sum(matrix_bytes(N, K, M) for _, N, K in LLAMA7B)
    return {
        "value": done_bytes / dt / 1e12, "unit": "TB/s", "cores": int(threads), "kind": "oracle",
        "sample": (f"layer 0 matrices {','.join(done)} ({layer_frac:.0%} of one layer), M={M}: "
                   f"numpy fp64 dequantize + BLAS product, {dt:.1f} s; "
                   f"equivalent {M * layer_frac / (dt * 32):.4f} tok/s for 32 layers"),
    }


def main():
    a = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {a.gpus}, WORLD_SIZE={world}); "
              "the multi-GPU layout is a design note, not a measured path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bit_weight_only_quantize_amd as w4
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    M = a.M

    # ---- weights: distinct seeded layers, quantized on the device
    layers = []
    for l in range(a.layers):
        mats = {}
        for name, N, K in LLAMA7B:
            W = synth.device_weights(N, K, 0.02, 0, f"llama7b.L{l}.{name}", dev)
            mats[name] = w4.quantize_pack(W, SCHEME)
            del W
        layers.append(mats)
    torch.cuda.synchronize()
    xs_host = {K: synth.activations_bf16(M, K, 0, f"llama7b.x{K}") for K in (4096, 11008)}
    xs = {K: torch.from_numpy(v.view(np.int16)).to(dev).view(torch.bfloat16) for K, v in xs_host.items()}
    ys = {name: torch.empty((M, N), dtype=torch.float32, device=dev) for name, N, _ in LLAMA7B}

    # per layer: Q/K/V share their input (one launch), O, gate/up share theirs (one
    # launch), down -- the launches a decode layer's data dependencies allow
    def step():
        for mats in layers:
            w4.gemv_multi_into([mats["wq"], mats["wk"], mats["wv"]], xs[4096],
                               [ys["wq"], ys["wk"], ys["wv"]])
            w4.gemv_into(mats["wo"], xs[4096], ys["wo"])
            w4.gemv_multi_into([mats["gate"], mats["up"]], xs[4096], [ys["gate"], ys["up"]])
            w4.gemv_into(mats["down"], xs[11008], ys["down"])

    def dominant():
        for mats in layers:
            w4.gemv_multi_into([mats["gate"], mats["up"]], xs[4096], [ys["gate"], ys["up"]])

    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        step()
        dominant()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()

    g_dom = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_dom):
        dominant()
    if a.dominant_only:
        for _ in range(a.warmup + a.steps):
            g_dom.replay()
        torch.cuda.synchronize()
        print(json.dumps({"dominant_only": True, "launches": a.layers * (a.warmup + a.steps)}))
        return
    g_step = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_step):
        step()

    # ---- timed region: whole step
    stream = torch.cuda.current_stream(dev)
    for _ in range(a.warmup):
        g_step.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(a.steps):
        g_step.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / a.steps

    # ---- dominant kernel (gate/up GEMV, 11008x4096): average launch duration
    for _ in range(2):
        g_dom.replay()
    torch.cuda.synchronize()
    reps = max(4, a.steps // 2)
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    d0.record(stream)
    for _ in range(reps):
        g_dom.replay()
    d1.record(stream)
    torch.cuda.synchronize()
    us_dom = d0.elapsed_time(d1) * 1e3 / (reps * a.layers)
    dom_bytes = group_bytes([(11008, 4096), (11008, 4096)], M)
    dom_gbs = dom_bytes / (us_dom * 1e-6) / 1e9

    step_bytes = a.layers * (group_bytes([(4096, 4096)] * 3, M) + matrix_bytes(4096, 4096, M)
                             + group_bytes([(11008, 4096)] * 2, M) + matrix_bytes(4096, 11008, M))
    tbs = step_bytes / (ms_step * 1e-3) / 1e12
    plan = None
    out = {
        "metric": METRIC, "value": round(tbs, 4), "unit": "TB/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "llama7b-shaped decode layer stack", "layers": a.layers, "M": M,
                   "scheme": SCHEME,
                   "matrices": "wq,wk,wv,wo 4096x4096; gate,up 11008x4096; down 4096x11008",
                   "weights": "seeded N(0,0.02) drawn on device", "activations": "bf16 N(0,1)"},
        "pct_of_hbm_peak": round(100 * tbs * 1e3 / HBM_PEAK_GBS, 2),
        "tok_per_s": round(M / (ms_step * 1e-3), 1),
        "step_bytes": step_bytes,
        "roofline": {"bound": "hbm",
                     "kernel": "gemv_wave_kernel (gate+up, 2 x 11008x4096 sym4_g128, one launch)",
                     "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dom_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_launch": dom_bytes, "avg_launch_us": round(us_dom, 3)},
    }
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(layers[0], xs_host, M, a.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
