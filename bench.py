#!/usr/bin/env python3
"""Benchmark of the grouped int4-dequant MoE layer on one MI355X.

One step = one moe_layer_forward call over T=2048 tokens of the
Qwen3.6-35B-A3B-shaped layer (d=2048, f=512, E=256 routed experts, top-8, one
shared expert, int4 groupwise-affine weights, 64 per group) with every input
already resident in HBM: top-k routing, scan/scatter/block map, the gate/up
grouped GEMM with SwiGLU and the down grouped GEMM with the weighted combine.

Prints one JSON line: tokens/s (value), the roofline of the dominant kernel
measured with HIP events recorded on the layer's stream inside the timed
region (only that kernel's two events there; every stage's figures come from
the same calls with all five events, run just before and untimed, and sit
beside it with the whole layer's), the T=1 and T=4 decode bandwidth, the other prefill workloads (the
512-token layer and the Zipf-skewed 8192-token prompt in 2048-token chunks),
and the CPU oracle timed on a bounded sample of the same workload (a
baseline, not a target).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

# kernel arguments in device memory, set before the HIP runtime starts (the
# package sets the same default on import); reported in the JSON line
os.environ.setdefault("HIP_FORCE_DEV_KERNARG", "1")

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix peak
HBM_PEAK_GBPS = 8000.0     # MI355X HBM3E peak
METRIC = "MoE-layer prefill tokens/s @T=2048 (% MFMA peak); T=1 HBM GB/s (% peak)"

# Bytes per launch of each GEMM kernel at T=2048, from two rocprofv3 --pmc passes
# (FETCH_SIZE, WRITE_SIZE) over this benchmark, scaled by what the same counters
# read for a plain 64 MiB device copy (FETCH_SIZE x 2.0, WRITE_SIZE x 1.0). They
# describe the kernels built from the sources with this digest; after any change
# to those sources the figure is stale and reported as null.
TRAFFIC_SOURCES = ("grouped_int4_dequant_amd/csrc/gemm_kernels.hip",
                   "grouped_int4_dequant_amd/csrc/prep_layout.h",
                   "grouped_int4_dequant_amd/csrc/rebuild_device.h",
                   "grouped_int4_dequant_amd/csrc/moe_internal.h",
                   "grouped_int4_dequant_amd/csrc/moe_api.hip",
                   "grouped_int4_dequant_amd/csrc/routing_kernels.hip")
TRAFFIC_DIGEST = "86eceafb1f07be89bdca7edde552d2d73258ab0b420ffdec30bb19f533486c4e"
TRAFFIC_BYTES = {"gate_up": (185227.0 * 2.0 + 18432.0) * 1024,
                 "down_combine": (85494.7 * 2.0 + 73728.0 + 37144.5 * 2.0 + 16385.1) * 1024}


def sources_digest():
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def hip_runtime():
    """The HIP runtime library already loaded into this process (by torch and
    the layer library alike), for event calls torch does not expose."""
    import ctypes
    path = next(line.split()[-1] for line in open("/proc/self/maps") if "libamdhip64" in line)
    return ctypes.CDLL(path)


class HipEvent:
    """A timing event created without the system-scope fence on record
    (hipEventDisableSystemFence): it only timestamps, so it neither writes back
    nor invalidates caches between the kernels it brackets."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, hip):
        import ctypes
        self._ct, self._hip = ctypes, hip
        h = ctypes.c_void_p()
        if hip.hipEventCreateWithFlags(ctypes.byref(h), ctypes.c_uint(self.DISABLE_SYSTEM_FENCE)) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        self.handle = h.value

    def record(self, stream):
        if self._hip.hipEventRecord(self._ct.c_void_p(self.handle), self._ct.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end):
        """Milliseconds from this event to `end`."""
        ms = self._ct.c_float()
        if self._hip.hipEventElapsedTime(self._ct.byref(ms), self._ct.c_void_p(self.handle),
                                         self._ct.c_void_p(end.handle)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--prewarm-ms", type=float, default=500.0,
                    help="untimed layer calls for this long before the warm-up steps (clock ramp-up)")
    ap.add_argument("--decode-steps", type=int, default=1000,
                    help="decode steps per token count (the 1000-step decode workload)")
    ap.add_argument("--cpu-tokens", type=int, default=2048, help="tokens in the CPU oracle sample (0: skip)")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="before the timed region, run a plain device copy of this many MiB three times "
                         "(a known-size kernel for calibrating hardware byte counters; 0: none)")
    ap.add_argument("--other-configs", type=int, default=1,
                    help="also time the 512-token layer and the skewed 8192-token prompt in 2048-token "
                         "chunks (0: skip)")
    ap.add_argument("--graph", type=int, default=1,
                    help="also time the layer captured into a HIP graph at T=2048 and T=512: the one-stream "
                         "capture and the concurrent capture (shared expert beside the routing) (0: skip)")
    ap.add_argument("--ablations", type=str, default="",
                    help="comma-separated token counts: also time the layer's ablation forms "
                         "(16-row work units; routing built on the host; weights expanded in memory "
                         "before the GEMMs) at each (e.g. 512,2048)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this layer has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import grouped_int4_dequant_amd as moe
    from grouped_int4_dequant_amd import binding as B
    from synth import moe_inputs as S

    moe.load()
    dev = torch.device("cuda", 0)
    cfg = S.CONFIGS[2]
    sh, T = cfg.shape, cfg.T
    p = S.make_problem(2)
    layer = moe.Layer.from_numpy(sh.d, sh.f, sh.E, sh.k, sh.f_sh, p.layer, device=dev)
    x = torch.from_numpy(p.x.view(np.int16)).view(torch.bfloat16).to(dev)
    lg = torch.from_numpy(p.logits).to(dev)
    y = torch.empty((T, sh.d), dtype=torch.float32, device=dev)
    ws = moe.alloc_workspace(moe.workspace_bytes(T, layer), dev)
    stream = torch.cuda.current_stream()

    lib = B.load()
    lib.moe_layer_forward_timed.argtypes = [
        B.ctypes.POINTER(B.MoeLayerT), B._P, B._P, B._I32, B._P, B._P, B._P, B.ctypes.c_size_t, B._P,
        B.ctypes.POINTER(B._P)]
    lib.moe_layer_forward_timed.restype = B.ctypes.c_int

    hip = hip_runtime()

    def make_events(n):
        return [HipEvent(hip) for _ in range(n)]

    def timed_call(evs):
        arr = (B._P * 5)(*[e.handle if e is not None else None for e in evs])
        st = lib.moe_layer_forward_timed(B.ctypes.byref(layer.c), x.data_ptr(), lg.data_ptr(), T,
                                         y.data_ptr(), None, ws.data_ptr(), ws.numel(),
                                         stream.cuda_stream, arr)
        if st != 0:
            raise RuntimeError(moe.status_string(st))

    if args.copy_mb > 0:
        n = args.copy_mb << 18
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    lib.moe_layer_forward.argtypes = [
        B.ctypes.POINTER(B.MoeLayerT), B._P, B._P, B._I32, B._P, B._P, B._P, B.ctypes.c_size_t, B._P]
    lib.moe_layer_forward.restype = B.ctypes.c_int
    fwd_args = (B.ctypes.byref(layer.c), x.data_ptr(), lg.data_ptr(), T, y.data_ptr(), None, ws.data_ptr(),
                ws.numel(), stream.cuda_stream)

    def plain_call():
        st = lib.moe_layer_forward(*fwd_args)
        if st != 0:
            raise RuntimeError(moe.status_string(st))

    # Pre-warm: the GPU's clocks ramp up over the first tens of milliseconds
    # of sustained work, so untimed calls run for a fixed wall time first;
    # then the W warm-up steps the contract names.
    t_end = time.perf_counter() + args.prewarm_ms * 1e-3
    while time.perf_counter() < t_end:
        for _ in range(20):
            plain_call()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        plain_call()
    torch.cuda.synchronize()
    # Stage breakdown (untimed): K calls with all five events, which the
    # library attaches to the kernel dispatches (start of the top-k, end of
    # each stage); each event costs the GPU about a microsecond.
    stages = ["topk", "scan", "gate_up", "down_combine"]
    stage_events = [make_events(5) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for evs in stage_events:
        timed_call(evs)
    torch.cuda.synchronize()
    stage_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    dur = {s: float(np.mean([evs[i].elapsed_time(evs[i + 1]) for evs in stage_events]))
           for i, s in enumerate(stages)}  # ms
    gpu_ms = float(np.mean([evs[0].elapsed_time(evs[4]) for evs in stage_events]))
    flops_tok_gu = 2 * 2 * sh.d * (sh.k * sh.f + sh.f_sh)  # gate/up: 2 flops x 2f x d per row
    flops_tok_dn = 2 * sh.d * (sh.k * sh.f + sh.f_sh)
    kern_flops = {"gate_up": flops_tok_gu * T, "down_combine": flops_tok_dn * T}
    dom = max(kern_flops, key=lambda s: dur[s])
    # Timed region: K layer calls back to back on one stream, with only the
    # dominant kernel's two events attached (the end of the stage before it
    # and its own end), measured live for the roofline.
    di = stages.index(dom)
    step_events = []
    for _ in range(args.steps):
        e = make_events(2)
        step_events.append([e[0] if i == di else e[1] if i == di + 1 else None for i in range(5)])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for evs in step_events:
        timed_call(evs)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    dom_ms = float(np.mean([evs[di].elapsed_time(evs[di + 1]) for evs in step_events]))
    # the same calls without events, for comparison
    t0 = time.perf_counter()
    for _ in range(args.steps):
        plain_call()
    torch.cuda.synchronize()
    plain_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ms_per_step = elapsed * 1e3 / args.steps

    achieved = kern_flops[dom] / (dom_ms * 1e-3) / 1e12
    layer_tflops = (flops_tok_gu + flops_tok_dn) * T / (ms_per_step * 1e-3) / 1e12
    touched_bytes = (sh.E + 1) * S.bytes_per_expert(sh)
    traffic = TRAFFIC_BYTES if sources_digest() == TRAFFIC_DIGEST else {}

    out = {
        "metric": METRIC,
        "value": T * args.steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup, "prewarm_ms": args.prewarm_ms,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "runtime_env": {"HIP_FORCE_DEV_KERNARG": os.environ.get("HIP_FORCE_DEV_KERNARG")},
        "config": {"workload": "moe_layer_prefill", "T": T, "d": sh.d, "f": sh.f, "E": sh.E, "k": sh.k,
                   "f_sh": sh.f_sh, "weights": "int4 groupwise-affine g=64 bf16 scale+bias",
                   "weights_layout": "prepared" if layer.c.prep else "original",
                   "inputs": "seeded synthetic (config 2 recipe)"},
        # achieved/frac/traffic: the dominant kernel (the contract's figure,
        # timed inside the timed region); "layer": the whole call's useful
        # FLOPs over its time per step, the figure the layer is judged by;
        # "kernels": every stage's share, from the untimed five-event calls
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / MFMA_PEAK_TFLOPS, "kernel_us": dom_ms * 1e3,
                     "traffic": traffic.get(dom),
                     "layer": {"achieved": layer_tflops, "frac": layer_tflops / MFMA_PEAK_TFLOPS,
                               "us_per_call": ms_per_step * 1e3,
                               "flops_per_call": (flops_tok_gu + flops_tok_dn) * T},
                     "kernels": {s: {"us": dur[s] * 1e3,
                                     **({"achieved": kern_flops[s] / (dur[s] * 1e-3) / 1e12,
                                         "frac": kern_flops[s] / (dur[s] * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS,
                                         "flops": kern_flops[s], "traffic": traffic.get(s)}
                                        if s in kern_flops else {})}
                                 for s in stages}},
        "stages_us": {s: dur[s] * 1e3 for s in stages},
        "layer": {"gpu_us_first_to_last_kernel": gpu_ms * 1e3, "us_per_call": ms_per_step * 1e3,
                  "us_per_call_without_events": plain_ms * 1e3,
                  "us_per_call_five_events": stage_ms * 1e3,
                  "useful_tflops": layer_tflops,
                  "mfma_frac": layer_tflops / MFMA_PEAK_TFLOPS,
                  "weight_gbps": touched_bytes / (ms_per_step * 1e-3) / 1e9},
    }

    out["router"] = bench_router(moe, S, torch, x, sh, args.steps)
    out["router_t1"] = bench_router_graph(moe, S, torch, x[:1].contiguous(), sh)
    if args.decode_steps > 0:
        out["decode_t1"] = bench_decode(moe, lib, B, S, torch, dev, stream, args.decode_steps, make_events)
        out["decode_t4"] = bench_decode(moe, lib, B, S, torch, dev, stream, args.decode_steps, make_events, T=4)
    if args.other_configs:
        out["other_configs"] = bench_prefill_configs(moe, S, torch, dev, args.steps)
    if args.graph:
        out["layer_graph"] = bench_graph(moe, S, torch, dev, args.steps)
    if args.ablations:
        out["ablations_us"] = bench_ablations(moe, lib, B, torch, layer, x, lg, y, ws, stream,
                                              [int(t) for t in args.ablations.split(",")],
                                              args.steps, args.warmup)
    del layer, x, lg, y, ws
    torch.cuda.empty_cache()
    if args.cpu_tokens > 0:
        out["cpu_baseline"] = cpu_baseline(p, args.cpu_tokens)
    print(json.dumps(out), flush=True)


def bench_router(moe, S, torch, x, sh, steps):
    """The router projection (logits = x W_r^T, bf16 in, fp32 out) over the
    benchmark's tokens with seeded N(0, 1/d) router weights: GPU time per
    call from events around back-to-back calls."""
    T = x.shape[0]
    w = S.draw_router(sh.E, sh.d, np.random.default_rng(1234))
    wt = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).to(x.device)
    lg = torch.empty((T, sh.E), dtype=torch.float32, device=x.device)
    for _ in range(5):
        moe.router_logits(x, wt, logits=lg)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        moe.router_logits(x, wt, logits=lg)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    return {"T": T, "d": sh.d, "E": sh.E, "us_per_call": us,
            "tflops": 2.0 * T * sh.d * sh.E / (us * 1e-6) / 1e12}


def bench_router_graph(moe, S, torch, x, sh, n=200, reps=3):
    """The router projection for a decode step's token (T = 1): n calls
    captured in a HIP graph and replayed, so the GPU time per call is the
    device's and not the host's call rate."""
    T = x.shape[0]
    w = S.draw_router(sh.E, sh.d, np.random.default_rng(1234))
    wt = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).to(x.device)
    lg = torch.empty((T, sh.E), dtype=torch.float32, device=x.device)
    for _ in range(5):
        moe.router_logits(x, wt, logits=lg)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for _ in range(n):
                moe.router_logits(x, wt, logits=lg)
    torch.cuda.current_stream().wait_stream(side)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * n)
    return {"T": T, "d": sh.d, "E": sh.E, "us_per_call": us, "weight_gbps": sh.E * sh.d * 2 / (us * 1e-6) / 1e9}


def bench_prefill_configs(moe, S, torch, dev, steps):
    """The other prefill workloads, each with inputs resident in HBM: the
    512-token layer (one moe_layer_forward call) and the 8192-token prompt
    with Zipf-skewed routing (one moe_prefill_chunked call over four
    2048-token chunks). GPU time per call from events around back-to-back
    calls after 300 ms of untimed calls; weight bytes count each chunk's touched experts
    (from the logits) plus the shared expert, read once per chunk."""
    res = {}
    for ci in (1, 3):
        cfg = S.CONFIGS[ci]
        sh, T, chunk = cfg.shape, cfg.T, cfg.chunk
        p = S.make_problem(ci)
        layer = moe.Layer.from_numpy(sh.d, sh.f, sh.E, sh.k, sh.f_sh, p.layer, device=dev)
        x = torch.from_numpy(p.x.view(np.int16)).view(torch.bfloat16).to(dev)
        lg = torch.from_numpy(p.logits).to(dev)
        y = torch.empty((T, sh.d), dtype=torch.float32, device=dev)
        ws = moe.alloc_workspace(moe.workspace_bytes(chunk or T, layer), dev)
        if chunk:
            def call():
                moe.prefill_chunked(layer, x, lg, chunk, y=y, ws=ws)
        else:
            def call():
                moe.layer_forward(layer, x, lg, y=y, ws=ws)
        n = max(1, steps if not chunk else steps // 4)
        # untimed calls for 300 ms first: building the inputs leaves the GPU
        # idle for seconds, and its clocks ramp up again only under load
        t_end = time.perf_counter() + 0.3
        while time.perf_counter() < t_end:
            for _ in range(5):
                call()
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            call()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / n
        c = chunk or T
        touched = [int(len(np.unique(np.argsort(-p.logits[i:i + c], axis=1, kind="stable")[:, :sh.k])))
                   for i in range(0, T, c)]
        wbytes = sum((t + 1) * S.bytes_per_expert(sh) for t in touched)
        flops = S.useful_flops_per_token(sh) * T
        res[cfg.name] = {"T": T, "chunk": chunk, "calls": n, "us_per_call": us,
                         "tokens_per_s": T / (us * 1e-6),
                         "useful_tflops": flops / (us * 1e-6) / 1e12,
                         "mfma_frac": flops / (us * 1e-6) / 1e12 / MFMA_PEAK_TFLOPS,
                         "touched_experts_per_chunk": touched, "weight_bytes": wbytes,
                         "weight_gbps": wbytes / (us * 1e-6) / 1e9,
                         "hbm_frac": wbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS}
        del layer, x, lg, y, ws
        torch.cuda.empty_cache()
    return res


def bench_graph(moe, S, torch, dev, steps):
    """GPU microseconds per call of the layer (configs 2 and 1) run eagerly,
    as a one-stream HIP graph, and as the concurrent graph whose shared-expert
    branch runs beside the routing (items of 96 and 48 rows), from events
    around back-to-back calls; the forms alternate twice and the lower figure
    of each is kept."""
    res = {}
    for ci in (2, 1):
        p = S.make_problem(ci)
        sh, T = p.shape, p.T
        layer = moe.Layer.from_numpy(sh.d, sh.f, sh.E, sh.k, sh.f_sh, p.layer, device=dev)
        x = torch.from_numpy(p.x.view(np.int16)).view(torch.bfloat16).to(dev)
        lg = torch.from_numpy(p.logits).to(dev)
        y = torch.empty((T, sh.d), dtype=torch.float32, device=dev)
        ws = moe.alloc_workspace(moe.workspace_bytes(T, layer), dev)
        forms = {"eager": lambda: moe.layer_forward(layer, x, lg, y=y, ws=ws)}
        graphs = {"graph_one_stream": moe.LayerGraph(layer, x, lg, y, ws=ws, concurrent=False),
                  "graph_concurrent_96": moe.LayerGraph(layer, x, lg, y, ws=ws, concurrent=True,
                                                        shared_unit_rows=96),
                  "graph_concurrent_48": moe.LayerGraph(layer, x, lg, y, ws=ws, concurrent=True,
                                                        shared_unit_rows=48)}
        for name, g in graphs.items():
            forms[name] = g.launch
        best = {}
        for _ in range(2):
            for name, fn in forms.items():
                for _ in range(5):
                    fn()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(steps):
                    fn()
                e1.record()
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / steps
                best[name] = min(us, best.get(name, us))
        res[f"T{T}_us_per_call"] = best
        for g in graphs.values():
            g.close()
        del layer, x, lg, y, ws
        torch.cuda.empty_cache()
    return res


def bench_ablations(moe, lib, B, torch, layer, x, lg, y, ws, stream, tokens, steps, warmup):
    """Wall-clock microseconds per call of each ablation form over the first T
    tokens of the benchmark input, calls back to back on one stream."""
    need = max(moe.ablation_workspace_bytes(T, layer, v) for T in tokens for v in moe.ABLATIONS)
    if ws.numel() < need:
        ws = moe.alloc_workspace(need, x.device)
    res = {}
    for T in tokens:
        if not 0 < T <= x.shape[0]:
            raise ValueError(f"ablation token count {T} outside 1..{x.shape[0]}")
        row = {}
        for name, variant in moe.ABLATIONS.items():
            args = (B.ctypes.byref(layer.c), x.data_ptr(), lg.data_ptr(), T, y.data_ptr(), None,
                    ws.data_ptr(), ws.numel(), stream.cuda_stream, variant)

            def call():
                st = lib.moe_layer_forward_ablation(*args)
                if st != 0:
                    raise RuntimeError(moe.status_string(st))
            for _ in range(warmup):
                call()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                call()
            torch.cuda.synchronize()
            row[name] = (time.perf_counter() - t0) * 1e6 / steps
        res[str(T)] = row
    return res


def bench_decode(moe, lib, B, S, torch, dev, stream, nsteps, make_events, T=1):
    """Decode steps of T tokens (1 or 4) with fresh logits and x, rotating over 4 device copies of the
    weights (about 1.8 GB, larger than the last-level cache) so repeated
    experts are not served from cache. Bytes per step are exact: the packed
    codes, scales and biases of the distinct experts touched plus the shared
    expert.

    The steps are captured into one HIP graph and replayed, so the GPU time
    per step is the device's (a decode loop would run captured steps too);
    the eager rate of back-to-back calls from Python is reported beside it.
    The replay's last output is checked against the eager one."""
    cfg = S.CONFIGS[4]
    sh = cfg.shape
    steps = list(S.decode_steps(T, steps=nsteps + 20))
    layers = [moe.Layer.from_numpy(sh.d, sh.f, sh.E, sh.k, sh.f_sh, steps[0].layer, device=dev, prepare=False)
              for _ in range(4)]
    xs = [torch.from_numpy(s.x.view(np.int16)).view(torch.bfloat16).to(dev) for s in steps]
    lgs = [torch.from_numpy(s.logits).to(dev) for s in steps]
    ys = [torch.empty((T, sh.d), dtype=torch.float32, device=dev) for _ in steps]
    ws = moe.alloc_workspace(moe.workspace_bytes(T, layers[0]), dev)
    per_expert = S.bytes_per_expert(sh)
    nbytes = []
    for s in steps:
        touched = len(np.unique(np.argsort(-s.logits, axis=1, kind="stable")[:, :sh.k]))
        nbytes.append((touched + 1) * per_expert)

    def run(i):
        moe.layer_forward(layers[i % 4], xs[i], lgs[i], y=ys[i], ws=ws)

    for i in range(20):
        run(i)
    torch.cuda.synchronize()
    # eager: back-to-back calls
    e0, e1 = make_events(2)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(20, 20 + nsteps):
        run(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / nsteps
    eager_gpu = e0.elapsed_time(e1) * 1e-3 / nsteps
    y_eager = ys[19 + nsteps].clone()
    # graph: the same steps captured once, replayed
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for i in range(20, 20 + nsteps):
                run(i)
    torch.cuda.current_stream().wait_stream(side)
    g.replay()
    torch.cuda.synchronize()
    reps = 3
    g0, g1 = make_events(2)
    g0.record(stream)
    for _ in range(reps):
        g.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    gpu = g0.elapsed_time(g1) * 1e-3 / (reps * nsteps)
    same = bool(torch.equal(ys[19 + nsteps], y_eager))
    b = float(np.mean(nbytes[20:]))
    return {"T": T, "steps": nsteps, "bytes_per_step": b,
            "gpu_us_per_step": gpu * 1e6, "eager_gpu_us_per_step": eager_gpu * 1e6,
            "wall_us_per_step": wall * 1e6, "graph_replay_matches_eager": same,
            "gbps_gpu": b / gpu / 1e9, "gbps_eager": b / eager_gpu / 1e9,
            "frac_hbm_gpu": b / gpu / 1e9 / HBM_PEAK_GBPS, "peak_gbps": HBM_PEAK_GBPS}


def _cpu_model():
    try:
        import subprocess
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name"):
                return line.split(":", 1)[1].strip()
    except Exception:
        pass
    return "unknown"


def _oracle_seconds(O, p, tokens, k, passes=1):
    """Wall seconds per pass of the oracle's layer computation (input
    generation excluded) on the listed tokens."""
    t0 = time.perf_counter()
    for _ in range(passes):
        O.moe_forward(p.layer, p.x, p.logits, k, tokens=tokens)
    return (time.perf_counter() - t0) / passes


def cpu_baseline(p, ntok):
    """The fp64 oracle as it stands, timed on this host: the headline value is
    the T=2048 workload (the first ntok tokens, whole passes until at least
    10 s), scaled to tokens/s, with BLAS on every core this process may run
    on. `configs` adds each workload on all cores and, for the 64- and
    512-token layers, the 2048-token chunk 1 of the skewed prompt and the
    decode step, on one thread."""
    from threadpoolctl import threadpool_limits
    from oracle import moe_oracle as O
    from synth import moe_inputs as S
    cores = len(os.sched_getaffinity(0))
    ntok = min(ntok, p.T)
    tok = np.arange(ntok)
    with threadpool_limits(limits=cores):
        passes, t0 = 0, time.perf_counter()
        while True:  # whole passes until at least 10 s of CPU work
            O.moe_forward(p.layer, p.x, p.logits, p.shape.k, tokens=tok)
            passes += 1
            dt = time.perf_counter() - t0
            if dt >= 10.0:
                break
        rows = {}
        for ci in (0, 1, 3):
            q = S.make_problem(ci)
            sec = _oracle_seconds(O, q, None, q.shape.k)
            rows[q.config.name] = {"T": q.T, "threads": cores, "seconds": sec, "tokens_per_s": q.T / sec}
        rows["prefill2048"] = {"T": p.T, "threads": cores, "seconds": dt / passes * p.T / ntok,
                               "tokens_per_s": ntok * passes / dt}
        dec = list(S.decode_steps(1, steps=41))
        checked = [dec[i] for i in (0, 20, 40)]
        sec = sum(_oracle_seconds(O, q, None, q.shape.k) for q in checked) / len(checked)
        rows["decode_t1"] = {"T": 1, "threads": cores, "seconds_per_step": sec, "steps_timed": 3}
    one = {}
    with threadpool_limits(limits=1):
        for ci in (0, 1):
            q = S.make_problem(ci)
            sec = _oracle_seconds(O, q, None, q.shape.k)
            one[q.config.name] = {"T": q.T, "threads": 1, "seconds": sec, "tokens_per_s": q.T / sec}
        q = S.make_problem(3)
        sec = _oracle_seconds(O, q, np.arange(2048, 4096), q.shape.k)
        one["skew8192_chunk1"] = {"T": 2048, "threads": 1, "seconds": sec, "tokens_per_s": 2048 / sec}
        sec = sum(_oracle_seconds(O, c, None, c.shape.k) for c in checked) / len(checked)
        one["decode_t1"] = {"T": 1, "threads": 1, "seconds_per_step": sec, "steps_timed": 3}
    what = f"all {p.T} tokens" if ntok == p.T else f"first {ntok} of {p.T} tokens"
    return {"value": ntok * passes / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": _cpu_model(), "affinity_cpus": cores,
            "sample": f"{what} of the T={p.T} workload, {passes} pass(es) of the fp64 numpy oracle on "
                      f"{cores} BLAS threads, each dequantising every expert the tokens touch "
                      f"({dt:.1f} s in total)",
            "configs_all_cores": rows, "configs_one_thread": one}


if __name__ == "__main__":
    main()
