#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE layer forward on one MI355X.

One step = one pass of the whole layer (router + top-k, permutation, grouped
SwiGLU expert FFN, weighted combine) over one batch of synthetic tokens, with
weights and inputs resident in HBM.  The default workload is the
Mixtral-8x7B-shaped bf16 layer (hidden 4096, 8 experts, top-2, inter 14336) at
decode batch T=64; T in {1, 8, 32} are measured too and reported under
"sweep".

Prints one JSON line: MoE-layer tokens/s (whole step), the roofline of the
dominant kernel (the gate/up weight-streaming GEMM, timed live with HIP events
recorded by the library on the launch stream), and the CPU oracle timed on a
bounded token sample on the host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published


# ------------------------------------------------------------------ byte accounting

def expert_bytes(wl, part: str) -> int:
    """Bytes of one expert's gate+up ('gu') or down ('d') weights, block scales included."""
    n = (2 if part == "gu" else 1) * wl.H * wl.I
    return {"f32": 4 * n, "bf16": 2 * n, "mxfp4": n // 2 + n // 32, "int4g32": n // 2 + 2 * (n // 32)}[wl.wfmt]


def step_bytes(wl, T: int, touched: int) -> dict:
    """Algorithmic HBM bytes of one step: every touched expert's weights read once, activations once."""
    a = 2 if wl.xdt == "bf16" else 4
    hb = 4 if wl.wfmt == "f32" else 2
    n = T * wl.k
    gu = touched * expert_bytes(wl, "gu") + T * wl.H * a + n * wl.I * hb
    down = touched * expert_bytes(wl, "d") + n * wl.I * hb + n * wl.H * 4
    route = wl.E * wl.H * a + T * wl.H * a + n * 8
    combine = n * wl.H * 4 + T * wl.H * a
    return {"gu": gu, "down": down, "route": route, "combine": combine,
            "total": gu + down + route + combine}


def cost_model(C_s: float, S_s: float) -> dict:
    """Seconds per token T = C + S (S: streaming term B / W, C: everything else) and the implied rate."""
    T_s = C_s + S_s
    return {"T_s": T_s, "tokens_per_s": 1.0 / T_s}


def streaming_time(bytes_: float, bandwidth: float) -> float:
    """S = B / W."""
    return bytes_ / bandwidth


# ------------------------------------------------------------------ measurement

def measure(layers, xs, outs, steps: int, warmup: int, trace: bool, max_traced: int = 32):
    """Time `steps` eager steps between two events; step i runs layer instance i % len(layers) on
    batch i % len(xs).  On up to `max_traced` evenly spaced steps the library also records events
    around the gate/up and down kernels (on the launch stream)."""
    import torch

    R, L = len(xs), len(layers)
    for i in range(warmup):
        layers[i % L].forward(xs[i % R], outs[i % R])
    stride = max(1, steps // max_traced) if trace else steps + 1
    traced = list(range(0, steps, stride)) if trace else []
    ev = {i: [torch.cuda.Event(enable_timing=True) for _ in range(3)] for i in traced}
    for trio in ev.values():  # create the underlying HIP events
        for e in trio:
            e.record()
    handles = {i: ctypes_arr(trio) for i, trio in ev.items()}
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record()
    for i in range(steps):
        layers[i % L].forward(xs[i % R], outs[i % R], trace=handles.get(i))
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)
    gu_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in traced]
    dn_ms = [ev[i][1].elapsed_time(ev[i][2]) for i in traced]
    return total_ms, wall, gu_ms, dn_ms, traced


def measure_graph(layers, xs, outs, steps: int, warmup: int):
    """The same step sequence with every step captured once as a HIP graph (one graph per step of
    a period of the layer and batch rotation) and replayed: exactly `steps` replays are timed.  The
    host launch overhead and inter-kernel gaps of the eager loop are gone.  Returns ms per step."""
    import math

    import torch

    R, L = len(xs), len(layers)
    period = L * R // math.gcd(L, R)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm every instance up off the capture
        for i in range(period):
            layers[i % L].forward(xs[i % R], outs[i % R])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for i in range(period):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            layers[i % L].forward(xs[i % R], outs[i % R])
        graphs.append(g)
    for i in range(warmup):
        graphs[i % period].replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        graphs[i % period].replay()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1)
    del graphs
    return ms / steps


def layer_instances(layer, n: int):
    """`n` layer instances with the same weights at distinct addresses (the first is `layer`): steps
    rotate through them so that the expert bytes of one step are not still in the 256 MB
    last-level cache from an earlier one."""
    from mixture_experts_layer_token_amd.layer import MoeLayer

    out = [layer]
    for _ in range(n - 1):
        out.append(MoeLayer(layer.H, layer.I, layer.E, layer.k, layer.fmt, layer.xdt, layer.w_router, layer.bias,
                            layer.packages.clone(), layer.pkg_stride, layer.shared, max_T=layer.max_T,
                            device=layer.device))
    return out


def ctypes_arr(trio):
    import ctypes

    arr = (ctypes.c_void_p * 3)(*[e.cuda_event for e in trio])
    return arr


def touched_per_batch(layer, xs, E):
    import torch

    out = []
    for x in xs:
        layer.forward(x)
        torch.cuda.synchronize()
        out.append(int((layer.counts.cpu().numpy() > 0).sum()))
    return out


def cpu_baseline(wl, xs_host, min_seconds: float = 10.0, max_tokens: int | None = None):
    """The oracle on whole batches of the timed workload (or on the first `max_tokens` tokens of one
    batch) until about `min_seconds` of host time is spent: routing, touched experts' SwiGLU FFN,
    shared expert, combine; expert weights generated untimed."""
    import oracle
    from synth import workloads as W

    wg, bias = W.router_weights(wl), W.router_bias(wl)
    cache = {}
    tokens, spent, batches = 0, 0.0, 0
    for i in range(64 * len(xs_host)):
        x = xs_host[i % len(xs_host)]
        if max_tokens is not None:
            x = np.ascontiguousarray(x[:max_tokens])
        lg = oracle.router_logits(wl.xdt, np.ascontiguousarray(x), wg, bias)
        ids, _ = oracle.topk_gates(lg, wl.k)
        experts = [None] * wl.E
        for e in sorted(set(ids.ravel().tolist())):
            if e not in cache:
                cache[e] = W.expert_weights(wl, 0, e)
            experts[e] = cache[e]
        shared = W.shared_weights(wl)
        t = time.perf_counter()
        oracle.moe_layer(wl.xdt, x, wg, bias, wl.k, wl.I, experts, shared, wl.I if shared else 0)
        spent += time.perf_counter() - t
        tokens += x.shape[0]
        batches += 1
        if spent >= min_seconds:
            break
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": tokens / spent, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d batch(es) of %d tokens of the timed workload (%d tokens), whole layer in fp64: "
                      "routing, top-k, touched experts' SwiGLU FFN, shared expert, combine; %.1f s"
                      % (batches, x.shape[0], tokens, spent)}


def profiled_traffic(name: str):
    """HBM bytes per launch measured by the profiler for a kernel, if its sources are unchanged since."""
    import hashlib

    p = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(p):
        return None
    rec = json.load(open(p))
    h = hashlib.sha256()
    for src in rec["sources"]:
        h.update(open(os.path.join(ROOT, src), "rb").read())
    return rec if h.hexdigest() == rec["sources_sha256"] else None


def run(args):
    import torch

    from synth import workloads as W

    from mixture_experts_layer_token_amd.layer import build_layer, to_device_act

    wl = W.WORKLOADS[args.workload]
    prefill = args.workload in PREFILL
    if args.T is None:
        args.T = wl.Ts[-1] if prefill else 64
    Ts = sorted(set([args.T] + (list(wl.Ts) if args.sweep and not prefill else [])))
    layer = build_layer(wl, max(Ts))
    n_inst = args.layers if args.layers is not None else (1 if prefill else DECODE_INSTANCES.get(wl.name, 8))
    layers = layer_instances(layer, n_inst)
    results = {}
    for T in Ts:
        xs_host = [W.activations(wl, T, 0, 1000 + r) for r in range(args.batches if not prefill else 2)]
        xs = [to_device_act(a, wl.xdt) for a in xs_host]
        outs = [torch.empty_like(x) for x in xs]
        touched = touched_per_batch(layer, xs, wl.E)
        steps = args.steps if T == args.T else max(20, args.steps // 4)
        if prefill:
            steps = min(steps, args.prefill_steps)
        total_ms, wall, gu_ms, dn_ms, traced = measure(layers, xs, outs, steps, min(args.warmup, steps), trace=True)
        graph_ms = (measure_graph(layers, xs, outs, steps, min(args.warmup, steps))
                    if args.graph and not prefill else None)
        b = [step_bytes(wl, T, touched[i % len(xs)]) for i in range(steps)]
        tot_bytes = sum(x["total"] for x in b)
        gu_bytes = sum(b[i]["gu"] for i in traced)  # bytes of the traced launches only
        dn_bytes = sum(b[i]["down"] for i in traced)
        ms = total_ms / steps
        results[T] = dict(T=T, ms_per_step=graph_ms if graph_ms is not None else ms,
                          tokens_per_s=T / ((graph_ms if graph_ms is not None else ms) / 1e3),
                          eager_ms_per_step=ms, eager_tokens_per_s=T * steps / (total_ms / 1e3),
                          gu_us=1e3 * float(np.mean(gu_ms)), down_us=1e3 * float(np.mean(dn_ms)),
                          gu_gbps=gu_bytes / (sum(gu_ms) / 1e3) / 1e9,
                          down_gbps=dn_bytes / (sum(dn_ms) / 1e3) / 1e9,
                          ffn_gbps=(gu_bytes + dn_bytes) / ((sum(gu_ms) + sum(dn_ms)) / 1e3) / 1e9,
                          step_gbps=tot_bytes / steps / ((graph_ms if graph_ms is not None else ms) / 1e3) / 1e9,
                          touched_mean=float(np.mean(touched)), gu_bytes_per_launch=gu_bytes / len(traced),
                          traced=len(traced),
                          steps=steps, wall_s=wall, xs_host=xs_host,
                          instances=n_inst)
    head = results[args.T]
    if prefill:
        return prefill_report(wl, args, head)
    out = {
        "metric": "MoE-layer tokens/s (decode, whole layer) + achieved HBM GB/s of the expert FFN",
        "value": round(head["tokens_per_s"], 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": head["steps"],
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.wfmt != "f32" else "f32",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights)",
        "config": {"workload": "%s decode" % wl.name, "T": args.T, "hidden": wl.H, "experts": wl.E, "top_k": wl.k,
                   "inter": wl.I, "weights": wl.wfmt, "activations": wl.xdt,
                   "launch": "hipGraph replay" if args.graph else "eager",
                   "layer_instances": head["instances"], "input_batches": args.batches},
        "eager": {"ms_per_step": round(head["eager_ms_per_step"], 5),
                  "tokens_per_s": round(head["eager_tokens_per_s"], 2), "steps": args.steps},
        "roofline": {"bound": "hbm", "kernel": "ffn_stream_kernel gate/up (weight-streaming grouped GEMM + SwiGLU)",
                     "achieved": round(head["gu_gbps"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(head["gu_gbps"] / HBM_PEAK_GBS, 4), "traffic": None,
                     "avg_launch_us": round(head["gu_us"], 3),
                     "algorithmic_bytes_per_launch": int(head["gu_bytes_per_launch"]),
                     "timed_launches": head["traced"]},
        "expert_ffn": {"gbps": round(head["ffn_gbps"], 1), "frac": round(head["ffn_gbps"] / HBM_PEAK_GBS, 4),
                       "gu_us": round(head["gu_us"], 3), "down_us": round(head["down_us"], 3),
                       "down_gbps": round(head["down_gbps"], 1)},
        "step_hbm_gbps": round(head["step_gbps"], 1),
        "sweep": [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()
                   if k in ("T", "tokens_per_s", "ms_per_step", "eager_ms_per_step", "gu_gbps", "down_gbps",
                            "ffn_gbps", "step_gbps", "touched_mean")} for r in results.values()],
    }
    if args.workload == "mixtral" and args.T == 64:
        rec = profiled_traffic("ffn_gu_mixtral_bf16_decode_T64_traffic.json")
        if rec is not None:
            out["roofline"]["traffic"] = int(rec["gu_traffic_bytes_per_launch"])
    # the pages' decode cost model T = C + S for this step: S = expert bytes / peak HBM bandwidth
    S = streaming_time(head["gu_bytes_per_launch"] + step_bytes(wl, args.T, int(round(head["touched_mean"])))["down"],
                       HBM_PEAK_GBS * 1e9)
    C = head["ms_per_step"] / 1e3 - S
    out["cost_model"] = {"S_ms_at_peak": round(S * 1e3, 4), "C_ms_residual": round(C * 1e3, 4)}
    if args.cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, head["xs_host"], args.cpu_seconds)
    return out


PREFILL = ("kimi",)
# decode layer instances per workload: enough that the bytes touched between two visits of one
# instance exceed the 256 MB last-level cache (gpt-oss touches ~53 MB per step at T = 1)
DECODE_INSTANCES = {"mixtral": 8, "gptoss": 24}
OFFLOAD = ("glm",)
# cache policies the offload run compares (the last one is the reported value): the plain LRU, and
# use counts halved every 32 lookup groups (4 steps of the 8 layers)
POLICIES = (("lru", 0), ("lfu_decay", 32))


def belady_hits(capacity: int, groups) -> int:
    """Hits of Belady's MIN over the same lookup groups (upper bound for any policy): a miss with a
    full cache evicts the resident key whose next use lies farthest ahead."""
    nxt = [dict() for _ in groups]  # per group: key -> index of its next group
    later = {}
    for g in range(len(groups) - 1, -1, -1):
        for key in groups[g]:
            nxt[g][key] = later.get(key, 1 << 60)
        for key in groups[g]:
            later[key] = g
    resident, nu, hits = set(), {}, 0
    for g, grp in enumerate(groups):
        cur = set(grp)
        for key in sorted(cur):
            if key in resident:
                hits += 1
            else:
                if len(resident) >= capacity:
                    victim = max((k for k in resident if k not in cur), key=lambda k: (nu[k], k))
                    resident.discard(victim)
                resident.add(key)
        for key in cur:
            nu[key] = nxt[g][key]
    return hits
PCIE_PEAK_GBS = 64.0  # PCIe 5.0 x16, one direction (the link figure the pages quote)


def run_offload(args):
    """256 decode steps through 8 layers whose experts live in pinned host memory (LRU cache in HBM)."""
    import torch

    from synth import workloads as W

    from mixture_experts_layer_token_amd import api
    from mixture_experts_layer_token_amd.layer import to_device_act
    from mixture_experts_layer_token_amd.offload import OffloadedModel

    wl = W.WORKLOADS["glm"]
    steps = min(args.offload_steps, wl.steps)
    Ts = [args.T] if args.T else [16, 1]
    model = OffloadedModel(wl, max(Ts), fill=False)
    runs, belady = {}, {}
    for T in Ts:
        xs = {(l, s): to_device_act(W.activations(wl, T, l, s), wl.xdt) for s in range(steps) for l in range(wl.layers)}
        # route every (step, layer) once to know which experts the run touches; only those packages are
        # generated into the bank (the others are never fetched); the timed run routes again itself
        touched = {l: set() for l in range(wl.layers)}
        ids = torch.empty((T, wl.k), dtype=torch.int32, device="cuda")
        gw = torch.empty((T, wl.k), dtype=torch.float32, device="cuda")
        for (l, s), x in xs.items():
            api.moe_route(x, model.wg[l], model.bias(l, s), wl.k, ids, gw)
            touched[l] |= set(ids.cpu().numpy().ravel().tolist())
        for l in range(wl.layers):
            model.fill(l, touched[l] - model.filled.get(l, set()))
            model.filled[l] = model.filled.get(l, set()) | touched[l]
        out = torch.empty((T, wl.H), dtype=torch.bfloat16, device="cuda")
        model.reset_cache()
        for l in range(wl.layers):  # warm the kernels through the full path (the cache is reset below)
            model.layer_forward(l, 0, xs[(l, 0)], out)
        # every policy with the FFN of the hits overlapping the copies, and the reported policy once
        # without the overlap
        variants = [(p, d, True) for p, d in POLICIES] + ([(*POLICIES[-1], False)] if T == Ts[0] else [])
        for policy, period, overlap in variants:
            model.reset_cache(policy, period, overlap)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for s in range(steps):
                for l in range(wl.layers):
                    model.layer_forward(l, s, xs[(l, s)], out, time_copies=True)
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
            st = model.cache.stats()
            plans = model.plans
            seen, cold = set(), 0
            per_epoch = {}
            for (s, l, n, h, m) in plans:
                ep = s // wl.rerank_every
                a = per_epoch.setdefault(ep, [0, 0])
                a[0] += h
                a[1] += n
            # compulsory misses: first lookup of each (layer, expert) key
            for (s, l, n, h, m), grp in zip(plans, model.groups):
                for key in grp:
                    if key not in seen:
                        seen.add(key)
                        cold += 1
            runs[(T, policy, overlap)] = {
                "T": T, "policy": policy if policy == "lru" else "%s/%d" % (policy, period), "steps": steps,
                "ffn_of_hits_during_copies": overlap,
                "layers": wl.layers, "wall_s": wall, "tokens_per_s": T * steps / wall,
                "hit_rate": st["hits"] / max(1, st["lookups"]),
                "hit_rate_cold_excluded": st["hits"] / max(1, st["lookups"] - cold),
                "hit_rate_per_epoch": [round(v[0] / max(1, v[1]), 4) for _, v in sorted(per_epoch.items())],
                "hit_rate_belady": belady.setdefault(T, belady_hits(model.capacity, model.groups)) / max(1, st["lookups"]),
                "lookups": st["lookups"], "misses": st["misses"], "bytes_fetched": st["bytes_fetched"],
                "copy_busy_s": model.copy_ms / 1e3,
                "link_gbps_busy": st["bytes_fetched"] / max(1e-9, model.copy_ms / 1e3) / 1e9,
                "link_gbps_wall": st["bytes_fetched"] / wall / 1e9}
    head = runs[(Ts[0], POLICIES[-1][0], True)]
    out = {
        "metric": "MoE-layer tokens/s (offloaded expert bank, decode) + expert-cache hit rate + link GB/s",
        "value": round(head["tokens_per_s"], 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": 1,
        "ms_per_step": round(head["wall_s"] / steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights quantized to int4g32)",
        "config": {"workload": wl.name, "T": Ts[0], "layers": wl.layers, "hidden": wl.H, "experts": wl.E,
                   "top_k": wl.k, "inter": wl.I, "cache_slots": model.capacity,
                   "cache_policy": head["policy"], "ffn_of_hits_during_copies": True,
                   "bank_bytes": wl.layers * wl.E * model.pkg_bytes},
        "roofline": {"bound": "link", "kernel": "hipMemcpyAsync host bank -> HBM slots (copy stream)",
                     "achieved": round(head["link_gbps_busy"], 2), "peak": PCIE_PEAK_GBS, "unit": "GB/s",
                     "frac": round(head["link_gbps_busy"] / PCIE_PEAK_GBS, 4), "traffic": None},
        "runs": [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()} for r in runs.values()],
    }
    model.close()
    return out



MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 / fp16 MFMA, published


def prefill_report(wl, args, head):
    """Prefill: the expert FFN is a dense grouped contraction, so the roofline is MFMA throughput."""
    T, n = args.T, args.T * wl.k
    gu_flops = 2.0 * n * (2 * wl.I) * wl.H
    dn_flops = 2.0 * n * wl.H * wl.I
    sh_flops = 2.0 * T * 3 * wl.H * wl.I if wl.shared else 0.0
    step_flops = gu_flops + dn_flops + sh_flops + 2.0 * T * wl.E * wl.H
    gu_tf = gu_flops / (head["gu_us"] * 1e-6) / 1e12
    dn_tf = dn_flops / (head["down_us"] * 1e-6) / 1e12
    out = {
        "metric": "MoE-layer tokens/s (prefill, whole layer incl. shared expert) + MFMA utilisation of the expert FFN",
        "value": round(head["tokens_per_s"], 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": head["steps"],
        "warmup": min(args.warmup, head["steps"]),
        "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16" if wl.wfmt == "int4g32" else "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights quantized to %s)" % wl.wfmt,
        "config": {"workload": "%s" % wl.name, "T": T, "hidden": wl.H, "experts": wl.E, "top_k": wl.k,
                   "inter": wl.I, "weights": wl.wfmt, "shared_expert": "bf16" if wl.shared else None},
        "roofline": {"bound": "mfma", "kernel": "routed gate/up grouped GEMM + SwiGLU",
                     "achieved": round(gu_tf, 1), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gu_tf / MFMA_PEAK_TFLOPS, 4), "traffic": None,
                     "avg_launch_us": round(head["gu_us"], 1), "flops_per_launch": gu_flops,
                     "timed_launches": head["traced"]},
        "expert_ffn": {"gu_us": round(head["gu_us"], 1), "down_us": round(head["down_us"], 1),
                       "down_tflops": round(dn_tf, 1)},
        "step_tflops": round(step_flops / (head["ms_per_step"] * 1e-3) / 1e12, 1),
    }
    if args.cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, head["xs_host"], args.cpu_seconds, max_tokens=args.cpu_tokens)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="mixtral", choices=["mixtral", "gptoss", "kimi", "glm"])
    ap.add_argument("--offload-steps", type=int, default=256)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="copy 1 GiB device-to-device before measuring (profiler byte-counter calibration)")
    ap.add_argument("--T", type=int, default=None, help="tokens per step (default 64 decode, 8192 prefill)")
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--cpu-tokens", type=int, default=16, help="prefill: oracle token sample")
    ap.add_argument("--batches", type=int, default=8, help="distinct input batches the steps rotate through")
    ap.add_argument("--layers", type=int, default=None,
                    help="decode: layer instances (same weights, distinct addresses) the steps rotate through")
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="decode: report the eager loop only (default: HIP graph replay, eager beside it)")
    ap.add_argument("--no-sweep", dest="sweep", action="store_false")
    ap.add_argument("--no-cpu-baseline", dest="cpu_baseline", action="store_false")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (expert parallelism is described, "
              "not implemented); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        # a plain device copy of known size, for calibrating the HBM byte counters of a profiler run
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    out = run_offload(args) if args.workload in OFFLOAD else run(args)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
