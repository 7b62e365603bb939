#!/usr/bin/env python3
"""Benchmarks of the W4A16 hot path on one MI355X.

Default workload (the one the headline metric is quoted on): a Llama-7B-shaped
decode layer stack. One step = one decode pass of M tokens (default 1) through
32 distinct layers, each with the projections Wq, Wk, Wv, Wo (4096x4096), gate,
up (11008x4096) and down (4096x11008), symmetric INT4 with 128-weight groups
(scale = absmax/7). Per layer: Q/K/V in one launch (shared input), O, and the
FFN through w4a16_ffn (h = bf16(gelu(gate x) * (up x)) feeds down): one
persistent launch for one token, gate+up / activation / down for several
(--ffn separate: gate+up and down as plain GEMV calls with their own inputs).

Other workloads (--workload): moe26b (Gemma-4-26B-A4B-shaped MoE FFN stack),
prefill (the two prefill GEMMs), llama13b (13B-shaped stack + tied head),
gemv1024 (the single 1024x1024 GEMV, cache-hot and cold).

Weights are seeded N(0, 0.02) drawn on the device and quantized with the
library's quantize_pack; activations are seeded bf16 N(0, 1). Every step is
captured once in a HIP graph and replayed; times come from HIP events on the
stream the kernels run on.

With no --workload every workload runs in turn, one JSON line each: the 7B
stack at M = 4 and 16, the 13B stack (+ head) at M = 1 and 8, the MoE stack at
M = 1 and 32, prefill, the single GEMV, the INT4 KV cache, and last the
headline line, the 7B stack at M = 1 with the CPU oracle timed beside it.
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
MFMA_BF16_PEAK_TFLOPS = 2500.0
LLAMA7B = [("wq", 4096, 4096), ("wk", 4096, 4096), ("wv", 4096, 4096), ("wo", 4096, 4096),
           ("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008)]
LLAMA13B = [("wq", 5120, 5120), ("wk", 5120, 5120), ("wv", 5120, 5120), ("wo", 5120, 5120),
            ("gate", 13824, 5120), ("up", 13824, 5120), ("down", 5120, 13824)]


GEMM_SOURCES = ("common.hpp", "launch.hpp", "gemm.hip")


def weight_bytes(scheme: str, N: int, K: int) -> int:
    """Stored bytes of one quantized N x K matrix (codes + scales + biases)."""
    if scheme == "sym4_g128":
        return N * K // 2 + N * (K // 128) * 4
    if scheme == "aff4_g64":
        return N * K // 2 + N * (K // 64) * 4
    return N * K + N * (K // 64) * 4


def gemv_bytes(scheme: str, shapes, M: int) -> int:
    """Algorithmic HBM bytes of one launch serving matrices that share x: weights,
    x once, every y."""
    K = shapes[0][1]
    return sum(weight_bytes(scheme, N, K) + M * N * 4 for N, _ in shapes) + M * K * 2


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="all",
                    choices=["all", "llama7b", "moe26b", "prefill", "llama13b", "gemv1024", "kv"],
                    help="all (default): every workload, one line each, the 7B M=1 headline last")
    ap.add_argument("--context", type=int, default=8192, help="kv: cached positions per layer")
    ap.add_argument("--M", type=int, default=None, help="decode tokens per step (one workload only)")
    ap.add_argument("--scheme", default=None, choices=["sym4_g128", "aff4_g64", "aff8_g64"],
                    help="weight scheme of the llama7b/llama13b stacks (default: sym4_g128 / aff4_g64)")
    ap.add_argument("--layers", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU oracle time budget, each of the all-cores and one-thread runs")
    ap.add_argument("--moe-path", default="layer", choices=["layer", "single", "launches"],
                    help="moe26b: w4a16_moe_layer with its default dispatch, w4a16_moe_layer with "
                         "the single launch for one token, or the router GEMV + "
                         "w4a16_moe_gemv_logits calls")
    ap.add_argument("--ffn", default="layer", choices=["layer", "single", "separate"],
                    help="llama stacks: the FFN through w4a16_ffn (h feeds down) with its default "
                         "launches, w4a16_ffn with the single persistent launch for one token, or "
                         "gate+up and down as separate GEMV calls with their own inputs")
    ap.add_argument("--kv-append", default="fused", choices=["fused", "separate"],
                    help="kv: the new K and V quantized inside the scores and weighted-sum launches "
                         "(w4_kv_scores_append, w4_kv_weighted_sum_append), or by w4_kv_append first")
    ap.add_argument("--calibrate", action="store_true",
                    help="first run a plain 1 GiB copy (for scaling HBM byte counters), then the workload")
    ap.add_argument("--dominant-only", action="store_true",
                    help="only replay the dominant kernel (for counter collection)")
    return ap.parse_args()


# ---------------------------------------------------------------- helpers
class Ctx:
    def __init__(self, a):
        import numpy as np
        import torch

        import bit_weight_only_quantize_amd as w4
        import synth

        self.np, self.torch, self.w4, self.synth, self.a = np, torch, w4, synth, a
        self.dev = torch.device("cuda:0")
        torch.cuda.set_device(self.dev)

    def quant(self, N, K, scheme, name, out=None, expert=None):
        W = self.synth.device_weights(N, K, 0.02, 0, name, self.dev)
        q = self.w4.quantize_pack(W, scheme, out=out, expert=expert)
        del W
        return q

    def quant_stack(self, E, N, K, scheme, name):
        """E experts of N x K drawn as one [E*N][K] matrix and quantized in one launch:
        the [E][N][...] stack is the same bytes as that matrix's storage."""
        q = self.w4.empty_quantized(scheme, N, K, num_experts=E)
        W = self.synth.device_weights(E * N, K, 0.02, 0, name, self.dev)
        flat = self.w4.QuantizedMatrix(scheme, E * N, K, q.codes.view(E * N, -1), q.scale.view(E * N, -1),
                                       None if q.bias is None else q.bias.view(E * N, -1))
        self.w4.quantize_pack(W, scheme, out=flat)
        del W
        return q

    def release(self):
        """Hand the previous workload's device memory back before the next one."""
        import gc
        gc.collect()
        self.torch.cuda.synchronize()
        self.torch.cuda.empty_cache()

    def x(self, M, K, name):
        host = self.synth.activations_bf16(M, K, 0, name)
        return host, self.torch.from_numpy(host.view(self.np.int16)).to(self.dev).view(self.torch.bfloat16)

    def graph(self, fn):
        torch = self.torch
        side = torch.cuda.Stream(self.dev)
        side.wait_stream(torch.cuda.current_stream(self.dev))
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream(self.dev).wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        return g

    def time_graph(self, g, reps, warmup):
        """ms per replay, HIP events on the stream the graph replays on."""
        torch = self.torch
        stream = torch.cuda.current_stream(self.dev)
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps


def base_line(a, metric, value, unit, ms, config, dtype="bf16"):
    return {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": a.steps,
            "warmup": a.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic",
            "config": config}


def hbm_roofline(kernel, nbytes, us, traffic=None):
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"bound": "hbm", "kernel": kernel, "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
            "bytes_per_launch": nbytes, "avg_launch_us": round(us, 3)}


def stream_copy(c, nbytes=1 << 30, reps=5):
    """A plain 1 GiB device-to-device copy timed on this machine in this run (reads and
    writes nbytes each): what a long streaming kernel reaches here, the second
    yardstick beside the 8 TB/s peak. Measured once per process."""
    if getattr(c, "_copy", None) is None:
        torch = c.torch
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=c.dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        s = e0.elapsed_time(e1) * 1e-3 / reps
        c._copy = {"TBps": round(2 * nbytes / s / 1e12, 4), "bytes_per_copy": 2 * nbytes,
                   "what": "torch copy_ of a 1 GiB fp32 buffer (read + write), HIP events, this box and run"}
        del src, dst
        torch.cuda.empty_cache()
    return c._copy


def gpu_clocks():
    """The engine and memory clock levels the driver marks current (sysfs; best effort)."""
    import glob
    out = {}
    for name in ("sclk", "mclk"):
        for f in sorted(glob.glob(f"/sys/class/drm/card*/device/pp_dpm_{name}")):
            try:
                cur = [l.split(":", 1)[1].replace("*", "").strip() for l in open(f) if l.rstrip().endswith("*")]
            except OSError:
                continue
            if cur:
                out[name] = cur[0]
                break
    return out or None


def with_copy_yardstick(c, out, tbs):
    """Attach the same-box copy rate and the decode line's share of it."""
    cp = stream_copy(c)
    out["stream_copy"] = cp
    out["pct_of_stream_copy"] = round(100 * tbs / cp["TBps"], 2)
    clk = gpu_clocks()
    if clk:
        out["gpu_clocks"] = clk
    return out


def calibration_copy(c, nbytes=1 << 30):
    """A plain elementwise copy of known size (reads and writes nbytes once each),
    run in the counter-collection mode so FETCH_SIZE / WRITE_SIZE can be scaled
    by what they read for it."""
    torch = c.torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=c.dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst
    return nbytes


def kernel_sources_digest(files):
    """sha256 over the sources a kernel is built from; a counter measurement is
    only reported while the kernel is unchanged since it was taken."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "bit_weight_only_quantize_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def library_digest():
    """sha256 over every library source file (name and bytes, sorted by name)."""
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(ROOT, "bit_weight_only_quantize_amd", "csrc")
    for f in sorted(os.listdir(d)):
        h.update(f.encode())
        with open(os.path.join(d, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(key):
    """HBM bytes per launch (or per layer) for `key` from the committed counter
    summary (a line `traffic <key>: <int> sources_sha256: <hex>`), or None when it
    is missing or any library source has changed since the counters were taken."""
    try:
        text = open(os.path.join(ROOT, "profiles", "hbm_counters.md")).read()
    except OSError:
        return None
    m = __import__("re").search(r"traffic " + __import__("re").escape(key) +
                                r":\s*(\d+)\s+sources_sha256:\s*([0-9a-f]{64})", text)
    if not m or m.group(2) != library_digest():
        return None
    return int(m.group(1))


# ---------------------------------------------------------------- dense decode stacks
def decode_stack(c: Ctx, shapes, scheme, layers, M, head=None, ffn="layer"):
    """Build `layers` distinct layers (and an optional head) and return the step
    and dominant-kernel closures plus byte counts."""
    w4 = c.w4
    mats = []
    for l in range(layers):
        mats.append({nm: c.quant(N, K, scheme, f"{scheme}.L{l}.{nm}") for nm, N, K in shapes})
    hq = c.quant(head[0], head[1], scheme, f"{scheme}.head") if head else None
    c.torch.cuda.synchronize()
    d = shapes[0][2]
    f = shapes[4][1]
    xh = {K: c.x(M, K, f"{scheme}.x{K}") for K in (d, f)}
    xs = {K: v[1] for K, v in xh.items()}
    ys = {nm: c.torch.empty((M, N), dtype=c.torch.float32, device=c.dev) for nm, N, _ in shapes}
    yh = c.torch.empty((M, head[0]), dtype=c.torch.float32, device=c.dev) if head else None
    if ffn in ("layer", "single"):
        # the FFN through w4a16_ffn: h = bf16(gelu(gate x) * (up x)) feeds down
        w4.ffn_set_path(w4.FFN_PATH_SINGLE_LAUNCH if ffn == "single" else w4.FFN_PATH_DEFAULT)
        ws = w4.ffn_workspace(mats[0]["down"], M, c.dev)
    else:
        # gate+up and down as separate GEMV calls with their own inputs; the
        # down projection's activations outgrow one CU's LDS at M = 16 (7B) and
        # M = 8 (13B): those launches split K across CUs through a workspace
        need = w4.gemv_workspace_bytes(mats[0]["down"], M)
        ws = c.torch.empty(need, dtype=c.torch.uint8, device=c.dev) if need else None

    def ffn_call(m):
        if ffn != "separate":
            w4.ffn(m["gate"], m["up"], m["down"], xs[d], workspace=ws, y=ys["down"])
        else:
            w4.gemv_multi_into([m["gate"], m["up"]], xs[d], [ys["gate"], ys["up"]])
            w4.gemv_ws_into(m["down"], xs[f], ys["down"], ws)

    def step():
        for m in mats:
            w4.gemv_multi_into([m["wq"], m["wk"], m["wv"]], xs[d], [ys["wq"], ys["wk"], ys["wv"]])
            w4.gemv_into(m["wo"], xs[d], ys["wo"])
            ffn_call(m)
        if hq is not None:
            w4.gemv_into(hq, xs[d], yh)

    hbuf = c.torch.empty((M, f), dtype=c.torch.bfloat16, device=c.dev)
    gu_ws = w4.ffn_gate_up_workspace(mats[0]["gate"], M, c.dev)

    def dominant():
        for m in mats:
            if ffn == "single" and M == 1:
                ffn_call(m)
            elif ffn == "layer":
                w4.ffn_gate_up(m["gate"], m["up"], xs[d], h=hbuf, workspace=gu_ws)
            else:
                w4.gemv_multi_into([m["gate"], m["up"]], xs[d], [ys["gate"], ys["up"]])

    per_layer = (gemv_bytes(scheme, [(d, d)] * 3, M) + gemv_bytes(scheme, [(d, d)], M)
                 + gemv_bytes(scheme, [(f, d)] * 2, M) + gemv_bytes(scheme, [(d, f)], M))
    step_bytes = layers * per_layer + (gemv_bytes(scheme, [(head[0], head[1])], M) if head else 0)
    if ffn == "layer":
        # gate and up weights, x, h written
        dom_bytes = 2 * weight_bytes(scheme, f, d) + 2 * M * d + 2 * M * f
    elif ffn == "single" and M == 1:
        # weights of all three, x, h written once and read by the down rows, y
        dom_bytes = (2 * weight_bytes(scheme, f, d) + weight_bytes(scheme, d, f) + 2 * d
                     + 2 * f * 2 + 4 * d)
    else:
        dom_bytes = gemv_bytes(scheme, [(f, d)] * 2, M)
    return mats, xh, step, dominant, step_bytes, dom_bytes


def host_cpu():
    """CPUs this process may run on, and the CPU model name."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return n, model


def _oracle_gemv_pass(layer, xs_host, M, budget_s, shapes, scheme):
    """Layer 0's matrices through the oracle, in order and again, until the budget;
    returns (bytes, matrices done, seconds)."""
    import oracle
    import torch
    host = {}
    for name, N, K in shapes:
        q = layer[name]
        bias = None if q.bias is None else q.bias.view(torch.int16).cpu().numpy().view("uint16")
        scale = q.scale.cpu().numpy() if scheme == "sym4_g128" else \
            q.scale.view(torch.int16).cpu().numpy().view("uint16")
        host[name] = (q.codes.cpu().numpy(), scale, bias)
    done_bytes, done, t0 = 0, 0, time.perf_counter()
    while time.perf_counter() - t0 <= budget_s:
        name, N, K = shapes[done % len(shapes)]
        oracle.gemv_reference(*host[name], scheme, xs_host[K])
        done_bytes += gemv_bytes(scheme, [(N, K)], M)
        done += 1
    return done_bytes, done, time.perf_counter() - t0


def cpu_baseline(layer, xs_host, M, budget_s, shapes, scheme, layers):
    """The oracle as it stands, on layer 0's matrices (host copies), until the
    budget: once with every thread its BLAS starts, once limited to one thread."""
    from threadpoolctl import threadpool_info, threadpool_limits
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    nproc, model = host_cpu()
    full = sum(gemv_bytes(scheme, [(N, K)], M) for _, N, K in shapes)

    def leg(cores):
        nb, done, dt = _oracle_gemv_pass(layer, xs_host, M, budget_s, shapes, scheme)
        frac = nb / full
        return {"value": nb / dt / 1e12, "unit": "TB/s", "cores": int(cores), "kind": "oracle",
                "sample": (f"layer 0's {len(shapes)} matrices ({','.join(n for n, _, _ in shapes)}) "
                           f"cycled {done} times ({frac:.2f} layers' bytes), M={M}: numpy fp64 "
                           f"dequantize + BLAS product, {dt:.1f} s; equivalent "
                           f"{M * frac / (dt * layers):.4f} tok/s for {layers} layers")}

    out = leg(threads)
    with threadpool_limits(limits=1):
        out["one_thread"] = leg(1)
    out["nproc"] = nproc
    out["cpu_model"] = model
    return out


def run_llama(c: Ctx, a, big: bool):
    shapes, scheme = (LLAMA13B, "aff4_g64") if big else (LLAMA7B, "sym4_g128")
    scheme = a.scheme or scheme
    layers = a.layers or (40 if big else 32)
    M = a.M or 1
    head = (152064, 5120) if big else None
    mats, xh, step, dominant, step_bytes, dom_bytes = decode_stack(c, shapes, scheme, layers, M, head,
                                                                   a.ffn)
    fused1 = a.ffn == "single" and M == 1
    g_dom = c.graph(dominant)
    if a.dominant_only:
        copy_bytes = calibration_copy(c)
        for _ in range(a.warmup + a.steps):
            g_dom.replay()
        c.torch.cuda.synchronize()
        return {"dominant_only": True, "launches": layers * (a.warmup + a.steps),
                "calibration_copy_bytes": copy_bytes}
    g_step = c.graph(step)
    ms = c.time_graph(g_step, a.steps, a.warmup)
    us_dom = c.time_graph(g_dom, max(4, a.steps // 2), 2) * 1e3 / layers
    tbs = step_bytes / (ms * 1e-3) / 1e12
    d, f = shapes[0][2], shapes[4][1]
    name = "llama13b-shaped decode layer stack + tied head" if big else "llama7b-shaped decode layer stack"
    out = base_line(a, METRIC, round(tbs, 4), "TB/s", ms, {
        "workload": name, "layers": layers, "M": M, "scheme": scheme,
        "matrices": ", ".join(f"{nm} {N}x{K}" for nm, N, K in shapes) + (f", head {head[0]}x{head[1]}" if head else ""),
        "launches_per_layer": "qkv (one launch), o, " + (
            "ffn (gate, up, gelu, down: one persistent launch)" if fused1 else
            "ffn (gate+up with gelu in the epilogue, down)" if a.ffn == "layer" and M == 1 else
            "ffn (gate+up, gelu, down" + (" in K parts + a summing launch" if c.w4.gemv_workspace_bytes(
                mats[0]["down"], M) else "") + ")" if a.ffn == "layer" else
            "gate+up (one launch), down with its own input" + (
                " (K parts on separate CUs, then a summing launch)"
                if c.w4.gemv_workspace_bytes(mats[0]["down"], M) else "")),
        "weights": "seeded N(0,0.02) drawn on device", "activations": "bf16 N(0,1)"})
    out["pct_of_hbm_peak"] = round(100 * tbs * 1e3 / HBM_PEAK_GBS, 2)
    with_copy_yardstick(c, out, tbs)
    out["tok_per_s"] = round(M / (ms * 1e-3), 1)
    out["step_bytes"] = step_bytes
    traffic = None
    if layers == (40 if big else 32) and scheme == ("aff4_g64" if big else "sym4_g128"):
        traffic = measured_traffic(f"{'llama13b' if big else 'llama7b'}_m{M}/ffn_gate_up")
    if fused1:
        traffic = None
        kname = f"ffn_kernel (gate+up 2 x {f}x{d}, gelu, down {d}x{f}, {scheme}, one launch)"
    elif a.ffn == "layer" and M == 1:
        kname = f"ffn_gate_up_kernel (gate+up 2 x {f}x{d} {scheme}, gelu epilogue, one launch)"
    elif a.ffn == "layer":
        kname = (f"w4a16_ffn_gate_up (gate+up 2 x {f}x{d} {scheme}, gelu: the gated skinny launch, "
                 "or where its tile pairs do not fit the GEMV launch + the activation launch)")
    else:
        kname = f"gate+up GEMV (2 x {f}x{d} {scheme}, one launch)"
    out["roofline"] = hbm_roofline(kname, dom_bytes, us_dom, traffic)
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(mats[0], {K: v[0] for K, v in xh.items()}, M,
                                           a.cpu_seconds, shapes, scheme, layers)
    return out


# ---------------------------------------------------------------- MoE
def run_moe(c: Ctx, a):
    torch, w4 = c.torch, c.w4
    E, D, F, Fs, k = 128, 2048, 768, 2048, 8
    layers = a.layers or 30
    M = a.M or 1
    L = []
    for l in range(layers):
        gate = c.quant_stack(E, F, D, "aff4_g64", f"moe.L{l}.gate")
        up = c.quant_stack(E, F, D, "aff4_g64", f"moe.L{l}.up")
        down = c.quant_stack(E, D, F, "aff4_g64", f"moe.L{l}.down")
        shared = [c.quant(Fs, D, "aff4_g64", f"moe.L{l}.sg"), c.quant(Fs, D, "aff4_g64", f"moe.L{l}.su"),
                  c.quant(D, Fs, "aff4_g64", f"moe.L{l}.sd")]
        router = c.quant(E, D, "aff8_g64", f"moe.L{l}.router")
        L.append((router, gate, up, down, shared))
    torch.cuda.synchronize()
    _, x = c.x(M, D, "moe.x")
    ids = [torch.empty((M, k), dtype=torch.int32, device=c.dev) for _ in range(layers)]
    wts = [torch.empty((M, k), dtype=torch.float32, device=c.dev) for _ in range(layers)]
    y = torch.empty((M, D), dtype=torch.float32, device=c.dev)
    one = M == 1
    if a.moe_path in ("layer", "single"):
        # router, top-k and the experts from x in one call: for one token three
        # launches (router GEMV, gate/up selecting its experts itself, down) or
        # the single launch; for several, router (+ top-k), bucketing, two
        # passes, combine
        single = a.moe_path == "single"
        w4.moe_layer_set_single_launch(single)
        ws = w4.moe_layer_workspace(M, k, E, D, F, Fs, c.dev)
        launches = ("one (router, top-k, shared and routed gate/up, down: work items of one persistent grid)"
                    if one and single else "router gemv, gate/up with the top-k inside, down" if one else
                    "router gemv, top-k, bucketing, gate/up, down, combine")

        def step():
            for l, (router, gate, up, down, shared) in enumerate(L):
                w4.moe_layer(router, gate, up, down, x, top_k=k, shared=shared, workspace=ws, y=y,
                             ids=ids[l], weights=wts[l])
    else:
        ws = torch.empty(w4.moe_workspace_bytes(M, k, E, D, F, Fs), dtype=torch.uint8, device=c.dev)
        logits = torch.empty((M, E), dtype=torch.float32, device=c.dev)
        launches = ("router gemv, gate/up with the top-k inside, down" if one else
                    "router gemv, top-k, bucketing, gate/up, down, combine")

        def step():
            for l, (router, gate, up, down, shared) in enumerate(L):
                w4.gemv_into(router, x, logits)
                w4.moe_gemv_logits(gate, up, down, x, logits, top_k=k, shared=shared, workspace=ws,
                                   y=y, ids=ids[l], weights=wts[l])

    g = c.graph(step)
    ms = c.time_graph(g, a.steps, a.warmup)
    expert_b = 3 * weight_bytes("aff4_g64", F, D)
    shared_b = 2 * weight_bytes("aff4_g64", Fs, D) + weight_bytes("aff4_g64", D, Fs)
    router_b = weight_bytes("aff8_g64", E, D)
    distinct = [len(set(i.cpu().numpy().ravel().tolist())) for i in ids]
    step_bytes = sum(router_b + u * expert_b + shared_b for u in distinct)
    tbs = step_bytes / (ms * 1e-3) / 1e12
    out = base_line(a, "MoE decode tok/s; HBM TB/s over the expert bytes read", round(M / (ms * 1e-3), 1),
                    "tok/s", ms, {
                        "workload": "gemma-4-26b-a4b-shaped MoE FFN stack", "layers": layers, "M": M,
                        "experts": E, "top_k": k, "d_model": D, "expert_ffn": F, "shared_ffn": Fs,
                        "scheme": "aff4_g64 experts/shared, aff8_g64 router",
                        "entry_point": {"layer": "w4a16_moe_layer", "single": "w4a16_moe_layer (single launch)",
                                        "launches": "w4a16_gemv + w4a16_moe_gemv_logits"}[a.moe_path],
                        "launches_per_layer": launches})
    out["hbm_TBps"] = round(tbs, 4)
    out["pct_of_hbm_peak"] = round(100 * tbs * 1e3 / HBM_PEAK_GBS, 2)
    with_copy_yardstick(c, out, tbs)
    out["distinct_experts_per_layer"] = sum(distinct) / len(distinct)
    out["step_bytes"] = step_bytes
    traffic = (measured_traffic(f"moe_m{M}/layer")
               if a.moe_path == "layer" and layers == 30 and M in (1, 32) else None)
    out["roofline"] = hbm_roofline(f"whole MoE layer ({launches})", step_bytes // layers, ms * 1e3 / layers,
                                   traffic)
    return out


# ---------------------------------------------------------------- INT4 KV cache
def run_kv(c: Ctx, a):
    """Decode over an INT4 KV cache (Shimmy article §3.2, TurboShimmy): per layer,
    append the new token's K and V vectors (quantize), the fused-dequant scores over
    the T + 1 cached keys and the weighted sum over the T + 1 cached values. By
    default the key append runs inside the scores launch and the value append
    inside the weighted-sum launch; `--kv-append separate` appends both first in a
    launch of their own. The weights are a fixed softmax of random logits: the
    softmax itself is not a library operation. Llama-7B-shaped: 32 layers, 32
    heads of 128."""
    torch, w4 = c.torch, c.w4
    layers = a.layers or 32
    Hq = Hkv = 32
    D = w4.KV_HEAD_DIM
    T = a.context
    Tn = T + 1
    gen = torch.Generator(device=c.dev)
    gen.manual_seed(0)
    L = []
    for _ in range(layers):
        kc, ks = w4.kv_cache(Hkv, Tn, c.dev)
        vc, vs = w4.kv_cache(Hkv, Tn, c.dev)
        for codes, scales in ((kc, ks), (vc, vs)):
            x = torch.randn((T, Hkv, D), generator=gen, device=c.dev)
            w4.kv_quantize(x, codes, scales, 0)
        L.append((kc, ks, vc, vs))
    knew = torch.randn((1, Hkv, D), generator=gen, device=c.dev)
    vnew = torch.randn((1, Hkv, D), generator=gen, device=c.dev)
    q = torch.randn((Hq, D), generator=gen, device=c.dev)
    p = torch.softmax(torch.randn((Hq, Tn), generator=gen, device=c.dev), dim=1).contiguous()
    scores = torch.empty((Hq, Tn), dtype=torch.float32, device=c.dev)
    out = torch.empty((Hq, D), dtype=torch.float32, device=c.dev)
    ws = torch.empty(w4.kv_weighted_sum_workspace_bytes(Hq, Tn), dtype=torch.uint8, device=c.dev)
    torch.cuda.synchronize()

    fused = a.kv_append == "fused"

    def step():
        for kc, ks, vc, vs in L:
            if fused:
                w4.kv_scores_append(q, knew, kc, ks, T, out=scores)
                w4.kv_weighted_sum_append(p, vnew, vc, vs, T, workspace=ws, out=out)
            else:
                w4.kv_append(knew, vnew, (kc, ks), (vc, vs), T)
                w4.kv_scores(q, kc, ks, Tn, out=scores)
                w4.kv_weighted_sum(p, vc, vs, workspace=ws, out=out)

    def dominant():
        for kc, ks, _, _ in L:
            if fused:  # rewrites position T with the same codes every time
                w4.kv_scores_append(q, knew, kc, ks, T, out=scores)
            else:
                w4.kv_scores(q, kc, ks, Tn, out=scores)

    cache_b = Hkv * Tn * (D // 2 + 4)                  # one of K or V: codes + scales
    scores_b = cache_b + Hq * D * 4 + Hq * Tn * 4        # + q read + scores written
    wsum_b = cache_b + Hq * Tn * 4 + Hq * D * 4          # + weights read + out written
    quant1_b = Hkv * (D * 4 + D // 2 + 4)                # one new vector per head: fp32 in, codes + scale out
    step_bytes = layers * (scores_b + wsum_b + 2 * quant1_b)
    dom_b = scores_b + quant1_b if fused else scores_b
    g = c.graph(step)
    ms = c.time_graph(g, a.steps, a.warmup)
    g_dom = c.graph(dominant)
    us_dom = c.time_graph(g_dom, max(4, a.steps // 2), 2) * 1e3 / layers
    tbs = step_bytes / (ms * 1e-3) / 1e12
    res = base_line(a, "INT4 KV decode (append + scores + weighted sum) HBM TB/s over the cache bytes read",
                    round(tbs, 4), "TB/s", ms, {
                        "workload": "llama7b-shaped INT4 KV cache decode, 32 layers", "layers": layers,
                        "heads_q": Hq, "heads_kv": Hkv, "head_dim": D, "context": Tn,
                        "cache_bytes": layers * 2 * cache_b,
                        "launches_per_layer": ("scores with the K append, weighted sum with the V append "
                                               "(+ chunk add)" if fused else
                                               "append K and V (one launch), scores, weighted sum (+ chunk add)")},
                    dtype="f32")
    res["pct_of_hbm_peak"] = round(100 * tbs * 1e3 / HBM_PEAK_GBS, 2)
    with_copy_yardstick(c, res, tbs)
    res["tok_per_s"] = round(1 / (ms * 1e-3), 1)
    res["step_bytes"] = step_bytes
    traffic = (measured_traffic("kv/scores_append" if fused else "kv/scores")
               if layers == 32 and T == 8192 else None)
    res["roofline"] = hbm_roofline(f"kv_scores_kernel ({Hq} heads x {Tn} positions, INT4 keys"
                                   + (", the new key appended in the same launch)" if fused else ")"),
                                   dom_b, us_dom, traffic)
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = kv_cpu_baseline(L[0], q, p, a.cpu_seconds, Tn)
    return res


def kv_cpu_baseline(layer, q, p, budget_s, Tn):
    """The oracle as it stands on layer 0's cache (host copies): scores and
    weighted sum repeated until the budget."""
    import oracle
    kc, ks, vc, vs = (t.cpu().numpy() for t in layer)
    qh, ph = q.cpu().numpy(), p.cpu().numpy()
    threads = os.cpu_count() or 1
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        pass
    n, t0 = 0, time.perf_counter()
    while True:
        oracle.kv_scores(qh, kc, ks)
        oracle.kv_weighted_sum(ph, vc, vs)
        n += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    nbytes = n * 2 * (kc.nbytes + ks.nbytes)
    return {"value": nbytes / dt / 1e12, "unit": "TB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"layer 0's K and V caches ({Tn} positions x 32 heads): numpy fp64 dequantize + "
                      f"matrix products, {n} passes in {dt:.1f} s"}


# ---------------------------------------------------------------- prefill
def run_prefill(c: Ctx, a):
    torch, w4 = c.torch, c.w4
    M = a.M or 2048
    res = {}
    for tag, N, K in (("gate_up", 11008, 4096), ("down", 4096, 11008)):
        q = c.quant(N, K, "sym4_g128", f"prefill.{tag}")
        _, X = c.x(M, K, f"prefill.X.{tag}")
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=c.dev)

        def fn(q=q, X=X, Y=Y):
            for _ in range(10):
                w4.gemm(q, X, Y)

        g = c.graph(fn)
        ms = c.time_graph(g, a.steps, a.warmup) / 10
        res[tag] = (ms, 2.0 * M * N * K)
    ms = sum(v[0] for v in res.values())
    fl = sum(v[1] for v in res.values())
    tfs = fl / (ms * 1e-3) / 1e12
    out = base_line(a, "Prefill W4A16 GEMM TFLOP/s (% of bf16 MFMA peak)", round(tfs, 2), "TFLOP/s", ms, {
        "workload": "prefill GEMMs 2048x4096 . 4096->11008 and 2048x11008 . 11008->4096",
        "M": M, "scheme": "sym4_g128"})
    for tag, (t, f) in res.items():
        out[f"{tag}_us"] = round(t * 1e3, 2)
        out[f"{tag}_TFLOPs"] = round(f / (t * 1e-3) / 1e12, 2)
    # Context, not the product: the vendor dense bf16 GEMM (hipBLASLt through
    # torch.matmul) on the same shapes with bf16 weights of the same layout
    # ([N][K], read transposed), i.e. what the matrix cores give these shapes
    # when no dequantization is involved and the weights are four times larger.
    dense = {}
    for tag, N, K in (("gate_up", 11008, 4096), ("down", 4096, 11008)):
        Xd = torch.randn(M, K, device=c.dev, dtype=torch.bfloat16)
        Wd = torch.randn(N, K, device=c.dev, dtype=torch.bfloat16)

        def fd(Xd=Xd, Wd=Wd):
            for _ in range(10):
                torch.matmul(Xd, Wd.t())

        gd = c.graph(fd)
        t = c.time_graph(gd, a.steps, a.warmup) / 10
        dense[tag] = {"us": round(t * 1e3, 2), "TFLOPs": round(2.0 * M * N * K / (t * 1e-3) / 1e12, 2)}
    out["dense_bf16_reference"] = dict(dense, what="torch.matmul (hipBLASLt) bf16 x bf16, same shapes, no dequantization")
    t, f = res["gate_up"]
    out["roofline"] = {"bound": "mfma", "kernel": "gemm_kernel (2048x4096 . 4096->11008, sym4_g128)",
                       "achieved": round(f / (t * 1e-3) / 1e12, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                       "unit": "TFLOP/s", "frac": round(f / (t * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                       "traffic": None, "flops_per_launch": f, "avg_launch_us": round(t * 1e3, 3)}
    busy = measured_mfma_busy("gemm_prefill_2048_mfma_counters.md", GEMM_SOURCES)
    if busy is not None:
        out["roofline"]["mfma_busy"] = busy
    return out


def measured_mfma_busy(profile, files):
    """Fraction of SIMD-cycles the matrix cores were busy in the gate/up GEMM, from a
    committed counter summary (`mfma_busy_gate_up: <f> sources_sha256: <hex>`), or
    None when it is missing or the kernel has changed since."""
    try:
        text = open(os.path.join(ROOT, "profiles", profile)).read()
    except OSError:
        return None
    m = __import__("re").search(r"mfma_busy_gate_up:\s*([0-9.]+)\s+sources_sha256:\s*([0-9a-f]{64})", text)
    if not m or m.group(2) != kernel_sources_digest(files):
        return None
    return float(m.group(1))


# ---------------------------------------------------------------- single GEMV
def run_gemv1024(c: Ctx, a):
    torch, w4 = c.torch, c.w4
    copies = 1024
    qs = [c.quant(1024, 1024, "aff4_g64", f"gemv1024.{i}") for i in range(copies)]
    _, x = c.x(1, 1024, "gemv1024.x")
    y = torch.empty((1, 1024), dtype=torch.float32, device=c.dev)
    hot = c.graph(lambda: [w4.gemv_into(qs[0], x, y) for _ in range(copies)])
    cold = c.graph(lambda: [w4.gemv_into(q, x, y) for q in qs])
    us_hot = c.time_graph(hot, a.steps, a.warmup) * 1e3 / copies
    us_cold = c.time_graph(cold, a.steps, a.warmup) * 1e3 / copies
    nb = gemv_bytes("aff4_g64", [(1024, 1024)], 1)
    out = base_line(a, "single 1024x1024 W4A16 GEMV latency (us)", round(us_cold, 3), "us", us_cold * 1e-3, {
        "workload": "gemv 1024x1024 aff4_g64, M=1", "cold": "1024 distinct copies (> MALL)"})
    out["higher_is_better"] = False
    out["hot_us"] = round(us_hot, 3)
    out["cold_GBs"] = round(nb / (us_cold * 1e-6) / 1e9, 1)
    return out


def main():
    a = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {a.gpus}, WORLD_SIZE={world}); "
              "the multi-GPU layout is a design note, not a measured path", file=sys.stderr)
        sys.exit(2)
    if a.workload == "all" and (a.M is not None or a.layers is not None or a.dominant_only):
        print("--M, --layers and --dominant-only apply to one --workload", file=sys.stderr)
        sys.exit(2)
    c = Ctx(a)
    if a.calibrate:
        calibration_copy(c)
    if a.workload != "all":
        print(json.dumps(run_one(c, a)), flush=True)
        return
    runs = [("llama7b", 4), ("llama7b", 16), ("llama13b", 1), ("llama13b", 8), ("moe26b", 1),
            ("moe26b", 32), ("prefill", None), ("gemv1024", None), ("kv", None)]
    for workload, M in runs:
        sub = argparse.Namespace(**dict(vars(a), workload=workload, M=M, no_cpu_baseline=True))
        print(json.dumps(run_one(c, sub)), flush=True)
        c.release()
    head = argparse.Namespace(**dict(vars(a), workload="llama7b", M=1))
    print(json.dumps(run_one(c, head)), flush=True)


def run_one(c, a):
    if a.workload in ("llama7b", "llama13b"):
        return run_llama(c, a, a.workload == "llama13b")
    if a.workload == "moe26b":
        return run_moe(c, a)
    if a.workload == "prefill":
        return run_prefill(c, a)
    if a.workload == "kv":
        return run_kv(c, a)
    return run_gemv1024(c, a)


if __name__ == "__main__":
    main()
