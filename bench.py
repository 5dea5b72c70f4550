#!/usr/bin/env python3
"""Benchmark of the fused MoE layer on one MI355X.

One step = one pass of the whole hot path over one batch: the routing/index
build and the forward pass ([fp8: per-token quantisation of x], gate-up GEMM,
SiLU-and-mul [+ fp8 requant], down GEMM, top-k weighted reduction), launched
through the C ABI on torch's current stream with every input already resident
in HBM.

Default workload: the largest single-GPU configuration, a DeepSeek-V3-shaped
layer in fp8 w8a8 (E=256, H=7168, I=2048, top-8, e4m3 weights with
per-output-channel fp32 scales, per-token e4m3 activations, bf16 output,
uniform softmax routing) at T=4096 tokens, with seeded synthetic weights and
tokens.  `value` is the layer's essential HBM bytes (weights and scales of the
experts that receive tokens + x + out + ids + weights) divided by the measured
time per layer, in GB/s.

W1/W2 are packed once into the kernels' MFMA-fragment order before timing
(moe_pack_weights, a load-time byte permutation); the CPU oracle reads the
row-major originals.

Printed: one JSON line (rank 0, N=1 only) with the timed-region figures, the
dominant kernel's roofline (HIP events recorded around it on the launch stream
inside the timed region), per-stage times, the workload's T sweep timed by
HIP-graph replay (median, p10, p90), the event and graph-launch overheads, the
attainable streaming-read rate of the device, and the CPU oracle timed on the
host as a baseline.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "us per MoE layer + achieved HBM GB/s (% of peak), T=1..4096 tokens, 1 GPU"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "mxfp8": 5000.0, "int8": 5000.0,   # int8: POP/s
                    "int4": 2500.0, "fp8b": 5000.0, "int8w": 2500.0}                                                   # bf16 MFMA
STAGES = ("quant_x", "gate_up", "act", "down", "reduce")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def layer_bytes_and_flops(wl, ids, T):
    """Essential HBM bytes of one layer call and its algorithmic flops."""
    import torch
    E, H, I = wl.E, wl.H, wl.I
    flat = ids.reshape(-1).to(torch.int64).cpu()
    valid = flat[(flat >= 0) & (flat < E)]
    active = int(torch.unique(valid).numel())
    bw = {"fp8": 1, "fp8b": 1, "mxfp8": 1, "int8": 1, "int4": 0.5, "int8w": 1}.get(wl.dtype, 2)
    # scales: fp32 per output channel (fp8, int8), one e8m0 byte per 32 weights (MX),
    # one fp32 per 128 weights (int4)
    per_expert = int(3 * H * I * bw) + {"fp8": (2 * I + H) * 4, "int8": (2 * I + H) * 4,
                                        "int8w": (2 * I + H) * 4,
                                        "mxfp8": 3 * H * I // 32,
                                        "int4": 3 * H * I // 128 * 4,
                                        "fp8b": 3 * H * I // (128 * 128) * 4}.get(wl.dtype, 0)
    P = flat.numel()
    nbytes = active * per_expert + T * H * 2 + T * H * 2 + P * 8
    flops = 6.0 * valid.numel() * H * I
    return nbytes, flops, active, int(valid.numel())


def stage_bytes(wl, active, P_valid, T, fused_reduce=False):
    """Algorithmic bytes each stage must move: its own inputs and outputs in
    their minimal form (weights and scales of the active experts once, the
    activations it reads, SiLU(gate)*up as bf16 or e4m3 codes, down rows as
    bf16); partial sums and padding rows are not counted.  fused_reduce: the
    down launch adds the top-k rows and writes the token rows itself."""
    E, H, I = wl.E, wl.H, wl.I
    mx = wl.dtype == "mxfp8"
    blk = wl.dtype == "fp8b"
    fp8 = wl.dtype in ("fp8", "int8") or mx or blk   # one-byte activation codes
    bw = 0.5 if wl.dtype == "int4" else (1 if fp8 or wl.dtype == "int8w" else 2)
    bx = 1 if fp8 else 2
    P = T * wl.k
    # per-row activation scales: 4 bytes (fp8) or one byte per 32 values (MX)
    xs = (H // 32 if mx else (H // 128 * 4 if blk else 4)) if fp8 else 0
    hs = (I // 32 if mx else (I // 128 * 4 if blk else 4)) if fp8 else 0
    w1s = ((2 * I * H // 32 if mx else (2 * I * H // 16384 * 4 if blk else 2 * I * 4)) if fp8
           else (2 * I * H // 128 * 4 if wl.dtype == "int4" else (2 * I * 4 if wl.dtype == "int8w" else 0)))
    w2s = ((H * I // 32 if mx else (H * I // 16384 * 4 if blk else H * 4)) if fp8
           else (H * I // 128 * 4 if wl.dtype == "int4" else (H * 4 if wl.dtype == "int8w" else 0)))
    return {
        "routing": P * 4 + P * 12,
        "quant_x": T * H * 2 + T * H + T * xs if fp8 else 0,
        "gate_up": int(active * (2 * I * H * bw + w1s)) + T * (H * bx + xs) + P_valid * I * bx,
        "act": P_valid * I * 4 + P_valid * (I * bx + hs),
        "down": int(active * (H * I * bw + w2s)) + P_valid * (I * bx + hs) +
                (T * H * 2 if fused_reduce else P_valid * H * 2),
        "reduce": 0 if fused_reduce else P_valid * H * 2 + T * H * 2,
    }


class Layer:
    """Buffers and launch of one layer at one token count."""

    def __init__(self, moe, wl, W, T, dtype, device="cuda"):
        import torch
        from moe_inputs import make_tokens
        self.moe, self.wl, self.W, self.T, self.dtype = moe, wl, W, T, dtype
        x, ids, w = make_tokens(wl, T, device=device)
        self.x, self.ids, self.w = x.contiguous(), ids.contiguous(), w.contiguous()
        E, H, I, k = wl.E, wl.H, wl.I, wl.k
        self.routing = moe.alloc_routing(T, k, E, H, I, dtype)
        self.ws = moe.alloc_workspace(T, k, E, H, I, dtype)
        self.out = torch.empty(T, H, dtype=torch.bfloat16, device=device)
        # a separate activation / requantisation launch exists only where the
        # gate-up GEMM leaves fp32 sums (workspace part "g")
        lay = moe.moe_workspace_layout(T, k, E, H, I, dtype)
        self.has_act = lay["g"] != 2 ** 64 - 1
        # one token: the down launch adds the top-k rows (no reduction launch)
        self.has_reduce = lay["y"] != 2 ** 64 - 1

    def run_routing(self):
        m, wl = self.moe, self.wl
        m.build_routing(self.ids, wl.E, wl.H, wl.I, self.routing, self.dtype)

    def run_forward(self, W=None):
        m, W = self.moe, (W or self.W)
        if self.dtype == "bf16":
            m.moe_forward_bf16(self.x, self.w, self.routing, W["w1"], W["w2"], self.ws, self.out)
        else:
            fwd = {"fp8": m.moe_forward_fp8, "mxfp8": m.moe_forward_mxfp8,
                   "int8": m.moe_forward_int8, "int4": m.moe_forward_int4,
                   "int8w": m.moe_forward_int8_w8a16,
                   "fp8b": m.moe_forward_fp8_block}[self.dtype]
            fwd(self.x, self.w, self.routing, W["w1"], W["w1_scale"], W["w2"], W["w2_scale"],
                self.ws, self.out)

    def run(self, W=None):
        """One layer: routing build + forward in one library call, which
        routes a decode batch (at most 64 pairs) inside the forward's first
        kernel."""
        m, W = self.moe, (W or self.W)
        m.route_forward(self.ids, self.x, self.w, self.routing, W, self.ws, self.out, self.dtype)


def stage_pass(layer, steps):
    """Untimed pass with HIP events around every stage (library stage hook)
    and around the routing build, which runs here as its own launch (the
    layer steps fold it into the forward's first kernel at decode).
    Each event record costs a few microseconds of stream time, so these
    steps are not the timed ones."""
    import torch
    moe = layer.moe
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(10)] for _ in range(steps)]
    rt = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for step_ev in ev:          # materialise the events before handing them over
        for e in step_ev:
            e.record()
    torch.cuda.synchronize()
    for i in range(steps):
        moe.moe_set_stage_events(ev[i])
        rt[i][0].record()
        layer.run_routing()
        rt[i][1].record()
        layer.run_forward()
    torch.cuda.synchronize()
    moe.moe_set_stage_events(None)
    stage_ms = {s: [] for s in STAGES}
    stage_ms["routing"] = [a.elapsed_time(b) for a, b in rt]
    for i in range(steps):
        for si, s in enumerate(STAGES):
            if layer.dtype in ("bf16", "int4", "int8w") and s == "quant_x":
                continue
            if s == "act" and not layer.has_act:   # formed in the gate-up epilogue
                continue
            if s == "reduce" and not layer.has_reduce:   # added by the down launch
                continue
            stage_ms[s].append(ev[i][2 * si].elapsed_time(ev[i][2 * si + 1]))
    return stage_ms


def timed_steps(layer, steps, warmup, dom_stage):
    """The timed region: `steps` eager steps (routing build + forward) with
    HIP events only around the dominant GEMM, recorded on the stream it is
    launched on by the library's stage hook."""
    import torch
    moe = layer.moe
    si = STAGES.index(dom_stage)
    for _ in range(warmup):
        layer.run()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    hooks = []
    for a, b in ev:
        a.record()
        b.record()
        h = [None] * 10
        h[2 * si], h[2 * si + 1] = a, b
        hooks.append(h)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        moe.moe_set_stage_events(hooks[i])
        layer.run()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    moe.moe_set_stage_events(None)
    return wall, [a.elapsed_time(b) for a, b in ev]


def graph_time_us(layer, weight_sets, reps=20, warmup=3, calls=10):
    """Per-layer time by HIP-graph replay: `calls` layer calls (routing build
    + forward) captured back to back in one graph, as the tuning guide's
    benchmark does, each on the next weight copy in turn so that no call
    finds the weights of the one before in the caches; the replay time
    divided by `calls`, median (and best) over `reps` replays.  Several calls
    per graph keep the host's packet submission ahead of the device, which a
    one-call graph does not: there the first kernels wait several
    microseconds each for their dispatch packets."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for W in weight_sets:
            layer.run(W)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(calls):
            layer.run(weight_sets[i % len(weight_sets)])
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b) * 1000.0 / calls)
    dec = statistics.quantiles(times, n=10)
    return {"median": statistics.median(times), "best": min(times), "p10": dec[0], "p90": dec[-1]}


def overheads_us(reps=50):
    """What the timing method itself costs: two HIP events recorded back to
    back on one stream (nothing between them), and the replay of a graph
    holding ten one-element kernels, per kernel (the floor of a chain of ten
    dependent launches in one graph, as the sweep replays them)."""
    import torch
    pair = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        b.record()
        b.synchronize()
        pair.append(a.elapsed_time(b) * 1000.0)
    t = torch.zeros(1, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        t.add_(1.0)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(10):
            t.add_(1.0)
    g.replay()
    torch.cuda.synchronize()
    tiny = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        b.synchronize()
        tiny.append(a.elapsed_time(b) * 1000.0 / 10)
    return {"event_pair_us": round(statistics.median(pair), 2),
            "tiny_kernel_in_graph_us": round(statistics.median(tiny), 2)}


def graph_read_us(moe, nbytes, calls=10, reps=20):
    """The layer's graph method applied to a plain read of `nbytes`: `calls`
    streaming reads (`moe_stream_read`, eight workgroups per compute unit)
    captured back to back in one graph, each of another buffer in turn, so
    that no read finds its bytes in the last-level cache; the replay time
    divided by `calls`, median over `reps` replays.  The time a single kernel
    needs to stream this many bytes, launch ramp included: the floor of a
    decode layer that reads its weights once."""
    import torch
    nbytes = max(16, nbytes // 16 * 16)
    nbuf = max(2, math.ceil(600e6 / nbytes) + 1)
    bufs = [torch.ones(nbytes, dtype=torch.uint8, device="cuda") for _ in range(nbuf)]
    sink = torch.empty(moe.moe_device_cu_count() * 8, dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for b in bufs:
            moe.moe_stream_read(b, sink)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(calls):
            moe.moe_stream_read(bufs[i % nbuf], sink)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b) * 1000.0 / calls)
    del g, bufs
    torch.cuda.empty_cache()
    return statistics.median(times)


def stream_read_ceiling(moe, gib=4, reps=10):
    """Attainable HBM read rate: the library's plain streaming-read kernel over
    a buffer far larger than the last-level cache (median of `reps` reads,
    HIP events around each)."""
    import torch
    buf = torch.ones(gib << 30, dtype=torch.uint8, device="cuda")
    nbytes = buf.numel()
    cus = moe.moe_device_cu_count()
    best = None
    for per_cu in (2, 4, 8):          # workgroups per compute unit (4 waves each)
        sink = torch.empty(cus * per_cu, dtype=torch.int32, device="cuda")
        moe.moe_stream_read(buf, sink)
        torch.cuda.synchronize()
        times = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            moe.moe_stream_read(buf, sink)
            b.record()
            b.synchronize()
            times.append(a.elapsed_time(b) * 1e-3)
        gbs = nbytes / statistics.median(times) / 1e9
        if best is None or gbs > best[0]:
            best = (gbs, per_cu)
    del buf
    torch.cuda.empty_cache()
    return {"kernel": "moe_stream_read (non-temporal 16-byte loads, 32 KiB chunks per workgroup)",
            "bytes": nbytes, "workgroups_per_cu": best[1], "GBs": round(best[0], 1),
            "frac_of_peak": round(best[0] / HBM_PEAK_GBS, 4)}


def tile_copy_rates(moe, row_bytes=8192, reps=4, runs=9):
    """Per-CU rate of token-tile copies into LDS, apart from any GEMM: the
    library's tile-copy kernel (one workgroup per CU, groups of 16 on one XCD
    sharing a 160-row tile, so the copies after the first pass hit L2) for
    each lane pattern; median of `runs` launches, HIP events around each."""
    import torch
    cus = moe.moe_device_cu_count()
    nbytes = max(1, cus // 128) * 8 * 160 * row_bytes
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(cus, dtype=torch.int32, device="cuda")
    moved = cus * reps * 160 * row_bytes
    names = {0: "contiguous 1 KiB (packed weights)", 1: "16 rows x 64 B, MFMA lane order",
             2: "16 rows x 64 B, a row per lane quad (the GEMMs' token chunks)"}
    out = {}
    for pattern in (0, 1, 2):
        moe.moe_tile_copy_read(pattern, buf, row_bytes, reps, sink)
        torch.cuda.synchronize()
        times = []
        for _ in range(runs):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            moe.moe_tile_copy_read(pattern, buf, row_bytes, reps, sink)
            b.record()
            b.synchronize()
            times.append(a.elapsed_time(b) * 1e-3)
        t = statistics.median(times)
        out[names[pattern]] = {"us": round(t * 1e6, 1), "GBs": round(moved / t / 1e9, 1),
                               "GBs_per_cu": round(moved / t / 1e9 / cus, 1)}
    del buf
    torch.cuda.empty_cache()
    return {"kernel": "moe_tile_copy_read (global->LDS copies of a 160-row tile, 16 workgroups per tile)",
            "row_bytes": row_bytes, "reps": reps, "cus": cus, "patterns": out}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# Whole-layer oracle cost (multiply-adds, 3*H*I per pair) above which the CPU
# baseline runs on a seeded token subset and is scaled to the full batch.
CPU_FULL_MACS = 6e10
CPU_SUBSET = 256


def cpu_baseline(wl, layer, W_host, dtype, reps=3):
    """The oracle as it stands (fp64 C, OpenMP over tokens) on the host's
    cores: the whole layer when that is a few seconds of work, else a seeded
    subset of CPU_SUBSET tokens (always the first and the last) whose time is
    scaled by T / CPU_SUBSET (the oracle's cost is linear in the tokens)."""
    import numpy as np
    import oracle
    x = layer.x.cpu()
    ids = layer.ids.cpu()
    w = layer.w.cpu()
    T = x.shape[0]
    rows = None
    if T * wl.k * 3.0 * wl.H * wl.I > CPU_FULL_MACS and T > CPU_SUBSET:
        g = np.random.default_rng(T)
        mid = sorted(g.choice(np.arange(1, T - 1), size=CPU_SUBSET - 2, replace=False).tolist())
        rows = [0] + mid + [T - 1]
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        if dtype == "bf16":
            oracle.forward_bf16(x, w, ids, W_host["w1"], W_host["w2"], rows=rows)
        else:
            fwd = {"fp8": oracle.forward_fp8, "mxfp8": oracle.forward_mxfp8,
                   "int8": oracle.forward_int8, "int4": oracle.forward_w4a16,
                   "int8w": oracle.forward_w8a16,
                   "fp8b": oracle.forward_fp8_block}[dtype]
            fwd(x, w, ids, W_host["w1"], W_host["w1_scale"], W_host["w2"], W_host["w2_scale"], rows=rows)
        times.append(time.perf_counter() - t0)
    sec = statistics.median(times)
    scale = 1.0 if rows is None else T / len(rows)
    return sec * scale, sec, (None if rows is None else len(rows)), oracle.num_threads()


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dsv3",
                    choices=["tiny", "mixtral", "qwen3", "qwen2", "dsv3", "dsv3b", "dsv3mx", "dsv3i8", "mixtral8",
                             "mixtral4"])
    ap.add_argument("--tokens", type=int, default=None,
                    help="tokens of the timed step (default: the workload's largest T)")
    ap.add_argument("--no-sweep", action="store_true", help="skip the graph-replay T sweep")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--once", action="store_true",
                    help="one untimed step only (for counter collection under a profiler)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy (3 times); under rocprofv3 "
                         "--pmc it gives the FETCH_SIZE/WRITE_SIZE a copy of known size reads")
    ap.add_argument("--ceiling", action="store_true",
                    help="measure only the attainable HBM read rate (the library's streaming-read "
                         "kernel over 4 GiB) and print it")
    ap.add_argument("--copy-rates", action="store_true",
                    help="measure only the per-CU rate of token-tile copies into LDS in three lane "
                         "patterns (the library's tile-copy kernel) and print it")
    ap.add_argument("--router", action="store_true",
                    help="measure the router top-k kernel (the step before the routing build) over "
                         "the workload's token grid instead of the layer")
    ap.add_argument("--router-gemm", action="store_true",
                    help="measure the precision-aware router GEMM (and GEMM + top-k) on the blog's "
                         "K=4096, N=192 sweep, or with --workload on that layer's router shape")
    ap.add_argument("--shared", type=int, default=0,
                    help="with --router: fused shared experts appended to each token's top-k")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the layer runs on a single MI355X and this build "
              "has no multi-GPU path (see the sharding design notes); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import mixture_experts_layer_lds_amd as moe
    from moe_inputs import WORKLOADS, make_weights

    torch.cuda.set_device(0)
    if args.copy_calibration:
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 3 x 1 GiB device copies done")
        return
    if args.ceiling:
        print(json.dumps({"metric": "attainable HBM read rate, 1 GPU", **stream_read_ceiling(moe)}),
              flush=True)
        return
    if args.copy_rates:
        print(json.dumps({"metric": "token-tile copy rate into LDS, 1 GPU", **tile_copy_rates(moe)}), flush=True)
        return
    wl = WORKLOADS[args.workload]
    if args.router_gemm:
        router_gemm_bench(moe, wl if "--workload" in sys.argv else None, args)
        return
    if args.router:
        router_bench(moe, wl, args)
        return
    dtype = wl.dtype if wl.dtype in ("fp8", "fp8b", "mxfp8", "int8", "int4", "int8w") else "bf16"
    T = args.tokens if args.tokens is not None else max(wl.Ts)
    log(f"[bench] workload={wl.name} T={T} dtype={dtype}: generating weights")
    W_rows = make_weights(wl, device="cuda")
    if wl.dtype == "f32":
        W_rows = {k: v.bfloat16().contiguous() for k, v in W_rows.items()}
    # one-time pre-pack of W1/W2 into MFMA-fragment order (load time, not timed)
    W = moe.pack_weights(W_rows, dtype)
    W_host = None if args.no_cpu_baseline else {k: v.cpu() for k, v in W_rows.items()}
    del W_rows
    torch.cuda.empty_cache()
    layer = Layer(moe, wl, W, T, dtype)

    if args.once:
        layer.run()
        torch.cuda.synchronize()
        log("[bench] one step done")
        return

    nbytes, flops, active, P_valid = layer_bytes_and_flops(wl, layer.ids, T)
    for _ in range(args.warmup):
        layer.run()
    stage_ms = stage_pass(layer, max(5, min(args.steps, 20)))
    sb = stage_bytes(wl, active, P_valid, T, fused_reduce=not layer.has_reduce)
    stages = {}
    for s, v in stage_ms.items():
        if v:
            avg = sum(v) / len(v)
            stages[s] = {"avg_us": round(avg * 1000.0, 2),
                         "algorithmic_GBs": round(sb[s] / (avg * 1e-3) / 1e9, 1) if sb[s] else None}
    dom = max(("gate_up", "down"), key=lambda s: stages[s]["avg_us"])
    log(f"[bench] timed region: {args.warmup} warmup + {args.steps} steps (events around {dom})")
    wall, dom_ms = timed_steps(layer, args.steps, args.warmup, dom)
    ms_per_step = wall * 1000.0 / args.steps
    gbs = nbytes / (ms_per_step * 1e-3) / 1e9
    dom_us = round(sum(dom_ms) / len(dom_ms) * 1000.0, 2)
    dom_bytes = sb[dom]
    dom_flops = 2.0 * P_valid * H_I(wl, dom)
    intensity = dom_flops / max(dom_bytes, 1)
    ridge = MFMA_PEAK_TFLOPS[dtype] * 1e12 / (HBM_PEAK_GBS * 1e9)
    if intensity < ridge:
        roof = {"kernel": f"grouped_gemm ({dom})", "bound": "hbm",
                "achieved": round(dom_bytes / (dom_us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    else:
        roof = {"kernel": f"grouped_gemm ({dom})", "bound": "mfma",
                "achieved": round(dom_flops / (dom_us * 1e-6) / 1e12, 1),
                "peak": MFMA_PEAK_TFLOPS[dtype], "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = counted_traffic(dom, wl.name, T)
    roof["algorithmic_bytes"] = dom_bytes
    roof["algorithmic_flops"] = dom_flops
    roof["avg_launch_us"] = dom_us
    roof["mfma_frac"] = round(dom_flops / (dom_us * 1e-6) / 1e12 / MFMA_PEAK_TFLOPS[dtype], 4)

    sweep = []
    if not args.no_sweep:
        for Ts in wl.Ts:
            lay = Layer(moe, wl, W, Ts, dtype)
            nb, fl, act_e, pv = layer_bytes_and_flops(wl, lay.ids, Ts)
            copies = 1
            if nb < 1e9:
                per_copy = sum(v.numel() * v.element_size() for v in W.values())
                copies = max(1, min(8, math.ceil(1e9 / nb), int(40e9 // per_copy)))
            sets = [W] + [{k: v.clone() for k, v in W.items()} for _ in range(copies - 1)]
            q = graph_time_us(lay, sets)
            med = q["median"]
            sweep.append({"T": Ts, "us_per_layer": round(med, 2), "p10_us": round(q["p10"], 2),
                          "p90_us": round(q["p90"], 2), "best_us": round(q["best"], 2),
                          "tokens_per_s": round(Ts / (med * 1e-6), 1),
                          "active_experts": act_e, "essential_MB": round(nb / 1e6, 2),
                          "GBs": round(nb / (med * 1e-6) / 1e9, 1),
                          "hbm_frac": round(nb / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                          "mfma_frac": round(fl / (med * 1e-6) / 1e12 / MFMA_PEAK_TFLOPS[dtype], 4),
                          "weight_copies": copies})
            del sets, lay
            torch.cuda.empty_cache()
            if nb < 1e9:
                # one plain streaming read of the layer's essential bytes, timed the same way
                floor = graph_read_us(moe, int(nb))
                sweep[-1]["read_floor_us"] = round(floor, 2)
                sweep[-1]["of_read_floor"] = round(floor / med, 4)
            log(f"[bench] sweep T={Ts}: {sweep[-1]['us_per_layer']} us, {sweep[-1]['GBs']} GB/s")
    over = overheads_us()
    ceiling = stream_read_ceiling(moe)
    log(f"[bench] streaming-read ceiling {ceiling['GBs']} GB/s")

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle on the host)")
        sec, sec_run, subset, cores = cpu_baseline(wl, layer, W_host, dtype)
        if subset is None:
            sample = (f"the full {wl.name} layer at T={T} ({T * wl.k} pairs), fp64 C oracle, "
                      f"OpenMP over tokens, median of 3 runs")
        else:
            sample = (f"a seeded subset of {subset} of the {T} tokens (first and last included) of the "
                      f"{wl.name} layer, fp64 C oracle, OpenMP over tokens, median of 3 runs of "
                      f"{sec_run:.2f} s, scaled by {T}/{subset} to the whole batch (extrapolated)")
        cpu = {"value": round(nbytes / sec / 1e9, 4), "unit": "GB/s", "cores": cores,
               "kind": "oracle", "us_per_layer": round(sec * 1e6, 1),
               "tokens_per_s": round(T / sec, 2), "extrapolated": subset is not None,
               "nproc": os.cpu_count(), "cpu_model": cpu_model(), "sample": sample}

    rec = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded N(0,1/sqrt(fan_in)) weights, N(0,1) tokens and router logits)",
        "config": {"workload": wl.label, "E": wl.E, "H": wl.H, "I": wl.I, "k": wl.k, "T": T,
                   "routing": wl.routing, "parallelism": "none (one GPU)"},
        "us_per_layer": round(ms_per_step * 1000.0, 2),
        "tokens_per_s": round(T / (ms_per_step * 1e-3), 1),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "mfma_frac": round(flops / (ms_per_step * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS[dtype], 4),
        "essential_bytes": nbytes,
        "algorithmic_flops": flops,
        "active_experts": active,
        "stages": stages,
        "stages_note": "per-stage HIP events from a separate untimed pass (events around every "
                       "stage); the timed region records events around the dominant GEMM only",
        "roofline": roof,
        "ceiling": ceiling,
        "overheads": over,
        "cpu_baseline": cpu,
        "sweep": sweep,
        "sweep_note": "HIP-graph replay of ten back-to-back layer calls (routing build + forward), "
                      "20 replays; per-layer median, p10, p90 and best",
    }
    print(json.dumps(rec), flush=True)


def router_bench(moe, wl, args):
    """Router top-k over fp32 logits [T][E]: per T of the workload's grid, the
    time per call of a 10-call HIP graph replay (HIP events around each replay
    on the launch stream, median of 20), i.e. the launch duration of the kernel
    in a chain of dependent launches.  (Events around single eager launches
    would time the host's launch path instead.)  Algorithmic bytes per call:
    the logits read once (T*E*4) and ids + weights written once
    (T*(k+shared)*8)."""
    import torch
    import oracle
    from moe_inputs import make_router_inputs
    k, ns = wl.k, args.shared
    sweep = []
    for T in wl.Ts:
        _, logits = make_router_inputs(wl, T)
        dev = logits.cuda()
        ids = torch.empty(T, k + ns, dtype=torch.int32, device="cuda")
        w = torch.empty(T, k + ns, dtype=torch.float32, device="cuda")
        nbytes = T * wl.E * 4 + T * (k + ns) * 8

        def call():
            moe.moe_router_topk(dev, k, True, ns, topk_ids=ids, topk_w=w)

        for _ in range(args.warmup):
            call()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            call()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for _ in range(10):
                call()
        times = []
        for _ in range(20):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) * 1000.0 / 10)
        gr_us = statistics.median(times)
        sweep.append({"T": T, "us_per_call": round(gr_us, 2), "algorithmic_bytes": nbytes,
                      "GBs": round(nbytes / (gr_us * 1e-6) / 1e9, 1),
                      "hbm_frac": round(nbytes / (gr_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)})
        log(f"[bench] router T={T}: {gr_us:.2f} us/call")
        del g
    cpu = None
    if not args.no_cpu_baseline:
        T = wl.Ts[-1]
        _, logits = make_router_inputs(wl, T)
        la = logits.numpy()
        oracle.router_topk(la, k, True, ns)
        t0 = time.perf_counter()
        reps = 5
        for _ in range(reps):
            oracle.router_topk(la, k, True, ns)
        sec = (time.perf_counter() - t0) / reps
        cpu = {"value": round(sec * 1e6, 1), "unit": "us per call", "cores": oracle.num_threads(),
               "kind": "oracle", "sample": f"T={T}, fp64 C oracle, mean of {reps} calls"}
    print(json.dumps({"metric": "router top-k us per call + algorithmic GB/s, 1 GPU",
                      "workload": wl.label, "E": wl.E, "k": k, "n_shared": ns,
                      "dtype": "f32", "data": "synthetic (the workload's seeded router logits)",
                      "sweep": sweep, "cpu_baseline": cpu}), flush=True)


ROUTER_GEMM_TS = (1, 16, 48, 96, 208, 512, 1024, 2048, 4096)   # the blog's Table 2 grid


def router_gemm_bench(moe, wl, args):
    """Precision-aware router GEMM, bf16 x [T][K] against the split fp32
    weights [N][K]: per T, the time per call of a HIP graph of C back-to-back
    calls, each on its own copy of x and of the weight pair, C chosen so that
    one replay touches at least 512 MB (no call finds its operands in the
    256 MB last-level cache from the previous replay); median of 20
    replays / C.  Timed both alone (scores) and followed by the router top-k
    (k of the workload, or 8) in the two-launch fused call.  Algorithmic
    bytes: the split pair (4 N K, the size of the fp32 weights), x (2 T K)
    and the scores (4 T N); MFMA work: two bf16 products, 4 T N K flops."""
    import torch
    import oracle
    from moe_inputs import router_hidden, router_weight
    if wl is None:
        name, N, K, Ts, k = "blog Router GEMM sweep shape", 192, 4096, ROUTER_GEMM_TS, 8
    else:
        name, N, K, Ts, k = wl.label + " (router)", wl.E, wl.H, wl.Ts, wl.k
    w = router_weight(N, K, seed=8).cuda()
    pair = moe.moe_router_split_weights(w)
    pair_bytes = pair.numel()
    sweep = []
    for T in Ts:
        xb = T * K * 2
        C = max(2, min(64, math.ceil(512e6 / (pair_bytes + xb))))
        pairs = [pair] + [pair.clone() for _ in range(C - 1)]
        x0 = router_hidden(T, K, seed=9 + T).cuda()
        xs = [x0] + [x0.clone() for _ in range(C - 1)]
        ws = torch.empty(max(moe.moe_router_workspace_bytes(T, N, K), 16), dtype=torch.uint8, device="cuda")
        sc = torch.empty(T, N, dtype=torch.float32, device="cuda")
        ids = torch.empty(T, k, dtype=torch.int32, device="cuda")
        tw = torch.empty(T, k, dtype=torch.float32, device="cuda")

        def gemm(c):
            moe.moe_router_gemm(xs[c], pairs[c], N, scores=sc, workspace=ws)

        def fused(c):
            moe.moe_router_gemm_topk(xs[c], pairs[c], N, k, topk_ids=ids, topk_w=tw, workspace=ws)

        res = {}
        for label, fn in (("gemm", gemm), ("gemm_topk", fused)):
            if label == "gemm_topk" and N > 256:
                continue
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                for c in range(C):
                    fn(c)
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for c in range(C):
                    fn(c)
            times = []
            for _ in range(20):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                g.replay()
                b.record()
                torch.cuda.synchronize()
                times.append(a.elapsed_time(b) * 1000.0 / C)
            res[label] = statistics.median(times)
            del g
        nbytes = pair_bytes + xb + T * N * 4
        flops = 4.0 * T * N * K
        us = res["gemm"]
        sweep.append({"T": T, "us_per_call": round(us, 2),
                      "us_per_call_with_topk": round(res["gemm_topk"], 2) if "gemm_topk" in res else None,
                      "algorithmic_bytes": nbytes, "GBs": round(nbytes / (us * 1e-6) / 1e9, 1),
                      "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                      "TFLOPs": round(flops / (us * 1e-6) / 1e12, 2),
                      "mfma_frac": round(flops / (us * 1e-6) / 1e12 / MFMA_PEAK_TFLOPS["bf16"], 4),
                      "copies": C})
        log(f"[bench] router gemm T={T}: {us:.2f} us/call ({sweep[-1]['GBs']} GB/s, "
            f"{sweep[-1]['TFLOPs']} TFLOP/s), with top-k {sweep[-1]['us_per_call_with_topk']}")
        del pairs, xs
        torch.cuda.empty_cache()
    cpu = None
    if not args.no_cpu_baseline:
        T = 64
        hi, lo = oracle.router_split(w.cpu().numpy())
        x = router_hidden(T, K, seed=9 + T)
        t0 = time.perf_counter()
        oracle.router_scores(x, hi, lo)
        sec = time.perf_counter() - t0
        cpu = {"value": round(sec * 1e6, 1), "unit": "us per call", "cores": oracle.num_threads(),
               "kind": "oracle", "sample": f"T={T}, N={N}, K={K}: fp64 C oracle, one call"}
    print(json.dumps({"metric": "router GEMM us per call (+ achieved GB/s and TFLOP/s), 1 GPU",
                      "workload": name, "N": N, "K": K, "dtype": "bf16 x bf16 (split fp32 weights)",
                      "data": "synthetic (N(0, 0.02) fp32 weights, bf16 hidden states with outlier channels)",
                      "sweep": sweep, "cpu_baseline": cpu}), flush=True)


def sources_hash(paths):
    """First 16 hex digits of the sha256 of the listed files, concatenated in order."""
    import hashlib
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counted_traffic(stage, workload, T):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    FETCH_SIZE/WRITE_SIZE summary (copy-calibrated), or None when no summary
    covers this kernel and workload, or when any source that decides the
    kernel (its file, the launch plan, the shared headers) changed since."""
    import glob
    import re
    for path in glob.glob(os.path.join(ROOT, "profiles", "traffic_*.md")):
        m = re.search(r"```json\s*(\{.*?\})\s*```", open(path).read(), re.S)
        if not m:
            continue
        rec = json.loads(m.group(1))
        if rec.get("kernel") != f"grouped_gemm ({stage})" or rec.get("workload") != workload \
                or rec.get("T") != T:
            continue
        srcs = rec.get("sources")
        if not srcs or not all(os.path.exists(os.path.join(ROOT, p)) for p in srcs):
            continue
        if sources_hash(srcs) != rec.get("sources_sha256_16"):
            return None
        return rec["traffic_bytes"]
    return None


def H_I(wl, stage):
    """Inner-product length x output width of one pair's GEMM in a stage."""
    return (2 * wl.I * wl.H) if stage == "gate_up" else (wl.H * wl.I)


if __name__ == "__main__":
    main()
