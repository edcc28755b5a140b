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

def measure(layers, xs, outs, steps: int, warmup: int, trace: bool, max_traced: int = 32, mode: str = "auto"):
    """Time `steps` eager steps between two events; step i runs layer instance i % len(layers) on
    batch i % len(xs).  On up to `max_traced` evenly spaced steps the library also records events
    around the gate/up and down kernels (on the launch stream)."""
    import torch

    R, L = len(xs), len(layers)
    for i in range(warmup):
        layers[i % L].forward(xs[i % R], outs[i % R], mode=mode)
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
        layers[i % L].forward(xs[i % R], outs[i % R], mode=mode, trace=handles.get(i))
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)
    gu_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in traced]
    dn_ms = [ev[i][1].elapsed_time(ev[i][2]) for i in traced]
    return total_ms, wall, gu_ms, dn_ms, traced


def measure_graph(layers, xs, outs, steps: int, warmup: int, mode: str = "auto"):
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
            layers[i % L].forward(xs[i % R], outs[i % R], mode=mode)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for i in range(period):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            layers[i % L].forward(xs[i % R], outs[i % R], mode=mode)
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


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _omp_threads(n: int | None):
    """Set the OpenMP thread count of this process (the oracle's parallel loops); returns the previous one."""
    import ctypes

    try:
        gomp = ctypes.CDLL("libgomp.so.1")
    except OSError:
        return None
    prev = gomp.omp_get_max_threads()
    if n is not None:
        gomp.omp_set_num_threads(n)
    return prev


def cpu_baseline(wl, xs_host, min_seconds: float = 10.0, max_tokens: int | None = None,
                 one_core_seconds: float = 3.0, one_core_tokens: int = 4):
    """The oracle on whole batches of the timed workload (or on the first `max_tokens` tokens of one
    batch) until about `min_seconds` of host time is spent: routing, touched experts' SwiGLU FFN,
    shared expert, combine; expert weights generated untimed.  Then the same on one core, on the
    first `one_core_tokens` tokens of the batches, for about `one_core_seconds`."""
    import oracle
    from synth import workloads as W

    wg, bias = W.router_weights(wl), W.router_bias(wl)
    cache = {}
    shared = W.shared_weights(wl)

    def timed(budget, cap):
        tokens, spent, batches = 0, 0.0, 0
        for i in range(64 * len(xs_host)):
            x = xs_host[i % len(xs_host)]
            if cap is not None:
                x = np.ascontiguousarray(x[:cap])
            lg = oracle.router_logits(wl.xdt, np.ascontiguousarray(x), wg, bias)
            ids, _ = oracle.topk_gates(lg, wl.k)
            experts = [None] * wl.E
            for e in sorted(set(ids.ravel().tolist())):
                if e not in cache:
                    cache[e] = W.expert_weights(wl, 0, e)
                experts[e] = cache[e]
            t = time.perf_counter()
            oracle.moe_layer(wl.xdt, x, wg, bias, wl.k, wl.I, experts, shared, wl.I if shared else 0)
            spent += time.perf_counter() - t
            tokens += x.shape[0]
            batches += 1
            if spent >= budget:
                break
        return tokens, spent, batches, x.shape[0]

    threads = _omp_threads(None) or int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    tokens, spent, batches, bt = timed(min_seconds, max_tokens)
    prev = _omp_threads(1)
    t1, s1, _, _ = timed(one_core_seconds, min(one_core_tokens, max_tokens or one_core_tokens))
    _omp_threads(prev)
    return {"value": tokens / spent, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "one_core": {"value": t1 / s1, "unit": "tokens/s", "cores": 1, "tokens": t1, "seconds": round(s1, 2)},
            "cpu_model": cpu_model(),
            "sample": "%d batch(es) of %d tokens of the timed workload (%d tokens), whole layer in fp64: "
                      "routing, top-k, touched experts' SwiGLU FFN, shared expert, combine; %.1f s"
                      % (batches, bt, tokens, spent)}


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
        total_ms, wall, gu_ms, dn_ms, traced = measure(layers, xs, outs, steps, min(args.warmup, steps), trace=True,
                                                       mode=args.mode)
        graph_ms = (measure_graph(layers, xs, outs, steps, min(args.warmup, steps), mode=args.mode)
                    if args.graph and not prefill else None)
        b = [step_bytes(wl, T, touched[i % len(xs)]) for i in range(steps)]
        tot_bytes = sum(x["total"] for x in b)
        gu_bytes = sum(b[i]["gu"] for i in traced)  # bytes of the traced launches only
        dn_bytes = sum(b[i]["down"] for i in traced)
        ms = total_ms / steps
        # the step sequence runs twice, as eager launches and as replayed HIP graphs (the same work,
        # timed the same way); the faster of the two is the step's figure
        use_graph = graph_ms is not None and graph_ms <= ms
        best = graph_ms if use_graph else ms
        results[T] = dict(T=T, ms_per_step=best, tokens_per_s=T / (best / 1e3),
                          launch="hipGraph replay" if use_graph else "eager", graph_ms_per_step=graph_ms,
                          eager_ms_per_step=ms, eager_tokens_per_s=T * steps / (total_ms / 1e3),
                          gu_us=1e3 * float(np.mean(gu_ms)), down_us=1e3 * float(np.mean(dn_ms)),
                          gu_gbps=gu_bytes / (sum(gu_ms) / 1e3) / 1e9,
                          down_gbps=dn_bytes / (sum(dn_ms) / 1e3) / 1e9,
                          ffn_gbps=(gu_bytes + dn_bytes) / ((sum(gu_ms) + sum(dn_ms)) / 1e3) / 1e9,
                          step_gbps=tot_bytes / steps / (best / 1e3) / 1e9,
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
                   "inter": wl.I, "weights": wl.wfmt, "activations": wl.xdt, "ffn_mode": args.mode,
                   "launch": head["launch"],
                   "layer_instances": head["instances"], "input_batches": args.batches},
        "eager": {"ms_per_step": round(head["eager_ms_per_step"], 5),
                  "tokens_per_s": round(head["eager_tokens_per_s"], 2), "steps": args.steps},
        "graph": ({"ms_per_step": round(head["graph_ms_per_step"], 5),
                   "tokens_per_s": round(args.T / (head["graph_ms_per_step"] / 1e3), 2), "steps": args.steps}
                  if head["graph_ms_per_step"] is not None else None),
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
                   if k in ("T", "tokens_per_s", "ms_per_step", "launch", "eager_ms_per_step", "graph_ms_per_step",
                            "gu_gbps", "down_gbps",
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
# prefetch heuristics the offload run compares: none, the next layer's experts of its previous step, its most
# used experts so far
PREFETCH = (None, "last", "popular")


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


def static_pins(model, groups_by_layer, per_layer: int):
    """Static pin: each layer's `per_layer` most used experts over a calibration window of lookups."""
    pins = {}
    for l, groups in groups_by_layer.items():
        cnt = np.zeros(model.E, np.int64)
        for g in groups:
            cnt[np.unique(g)] += 1
        pins[l] = np.sort(np.argsort(-cnt, kind="stable")[:per_layer])
    return pins


def run_offload_compressed(args):
    """The GLM-shaped offload run with bf16 experts (four layers), plain and with both tiers
    compressed (the bank and the HBM slots hold exponent-window blobs, decoded into a working pool
    before each FFN pass), in the same HBM budget: 25% of the bank's plain packages."""
    import torch

    from synth import workloads as W

    from mixture_experts_layer_token_amd import api
    from mixture_experts_layer_token_amd.layer import pack_bank, to_device_act
    from mixture_experts_layer_token_amd.offload import OffloadedModel

    # four of the GLM-shaped layers: their bf16 bank (48 GB) is as much page-locked host memory as the
    # box grants one process with room to spare (eight layers, 97 GB, are refused)
    wl = W.WORKLOADS["glm"].with_(wfmt="bf16", name="glm-offload-bf16", layers=4)
    steps = min(args.offload_steps, wl.steps)
    Ts = [args.T] if args.T else [16, 1]
    raw_bytes = api.moe_package_bytes(wl.H, wl.I, "bf16")
    raw_stride = (raw_bytes + 255) // 256 * 256
    slots_raw = int(wl.cache_frac * wl.layers * wl.E)
    budget = slots_raw * raw_stride  # HBM for expert weights, the same in both runs
    # blob slot: the largest blob of a sample of experts (one per layer and a few more), plus 0.3%;
    # the fill refuses any blob that does not fit
    sample = [pack_bank(wl, l, [e])[0, :raw_bytes] for l in range(wl.layers) for e in (0, 97, 211)]
    largest = max(api.moe_compress_package(p).size for p in sample)
    blob_bytes = (int(largest * 1.003) + 255) // 256 * 256
    runs, belady, touched_all = [], {}, {}
    policies = (("lfu_decay", 32), ("lru", 0))
    work_slots = 16  # plain packages the compressed run decodes into, a layer's experts a group at a time
    for compressed in (False, True):
        cap_max = slots_raw if not compressed else (budget - min(wl.E, min(Ts) * wl.k, work_slots) * raw_stride) // blob_bytes
        model = OffloadedModel(wl, max(Ts), capacity=cap_max, fill=False, compressed=compressed,
                               blob_bytes=blob_bytes if compressed else None, work_slots=work_slots)
        for T in Ts:
            xs = {(l, s): to_device_act(W.activations(wl, T, l, s), wl.xdt) for s in range(steps)
                  for l in range(wl.layers)}
            if T not in touched_all:
                touched = {l: set() for l in range(wl.layers)}
                ids = torch.empty((T, wl.k), dtype=torch.int32, device="cuda")
                gw = torch.empty((T, wl.k), dtype=torch.float32, device="cuda")
                for (l, s), x in xs.items():
                    api.moe_route(x, model.wg[l], model.bias(l, s), wl.k, ids, gw)
                    touched[l] |= set(ids.cpu().numpy().ravel().tolist())
                touched_all[T] = touched
            for l in range(wl.layers):
                model.fill(l, touched_all[T][l] - model.filled.get(l, set()))
                model.filled[l] = model.filled.get(l, set()) | touched_all[T][l]
            # compressed: the working pool takes min(E, T k, work_slots) plain packages of the budget
            n_work = min(wl.E, T * wl.k, work_slots)
            cap = slots_raw if not compressed else (budget - n_work * raw_stride) // blob_bytes
            out = torch.empty((T, wl.H), dtype=torch.bfloat16, device="cuda")
            model.reset_cache(capacity=cap, prefetch=None)
            for l in range(wl.layers):  # warm the kernels through the full path
                model.layer_forward(l, 0, xs[(l, 0)], out)
            for policy, period in policies:
                r = offload_variant(model, wl, T, steps, xs, out, policy, period, True, None, None, belady)
                r["tiers"] = "compressed" if compressed else "plain"
                r["working_pool_slots"] = n_work if compressed else 0
                runs.append(r)
                print("offload %s T=%d %s: %.1f tokens/s, hit %.4f, %d slots" % (
                    r["tiers"], T, r["policy"], r["tokens_per_s"], r["hit_rate"], r["cache_slots"]), flush=True)
            del xs
        if compressed:
            blob_sizes = model.blob_sizes[model.blob_sizes > 0]
            dec = time_decoder(model, min(64, model.n_work))
        model.close()
        del model
    head = max((r for r in runs if r["T"] == Ts[0] and r["tiers"] == "compressed"), key=lambda r: r["tokens_per_s"])
    plain = max((r for r in runs if r["T"] == Ts[0] and r["tiers"] == "plain"), key=lambda r: r["tokens_per_s"])
    return {
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
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) bf16 weights)",
        "config": {"workload": wl.name, "T": Ts[0], "layers": wl.layers, "hidden": wl.H, "experts": wl.E,
                   "top_k": wl.k, "inter": wl.I, "tiers": "compressed (bank and HBM slots)",
                   "hbm_budget_bytes": budget, "cache_policy": head["policy"],
                   "reported": "compressed tiers, the faster policy at this T; plain tiers beside"},
        "vs_plain_tiers": round(head["tokens_per_s"] / plain["tokens_per_s"], 4),
        "compression": {"raw_bytes": raw_bytes, "blob_slot_bytes": blob_bytes,
                        "blob_bytes_mean": float(blob_sizes.mean()), "blob_bytes_max": int(blob_sizes.max()),
                        "ratio_mean": round(float(blob_sizes.mean()) / raw_bytes, 5),
                        "ratio_slot": round(blob_bytes / raw_bytes, 5), "experts": int(blob_sizes.size)},
        "roofline": {"bound": "link", "kernel": "hipMemcpyAsync host bank -> HBM slots (copy stream)",
                     "achieved": round(head["link_gbps_busy"], 2), "peak": PCIE_PEAK_GBS, "unit": "GB/s",
                     "frac": round(head["link_gbps_busy"] / PCIE_PEAK_GBS, 4), "traffic": None},
        "decoder_roofline": dec,
        "runs": [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()} for r in runs],
    }


def time_decoder(model, n: int) -> dict:
    """HBM roofline of the package decoder on n blobs of the model's bank (decoded into its working
    pool in one launch)."""
    import torch

    keys = [(l, e) for l in range(model.L) for e in range(model.E) if model.blob_sizes[l, e] > 0][:n]
    for i, (l, e) in enumerate(keys):
        model.pool[i].copy_(torch.from_numpy(model.package(l, e).copy()))
    sizes = [int(model.blob_sizes[l, e]) for l, e in keys]
    return decoder_roofline(model.pool, model.stride, model.work, model.raw_stride, sizes, model.raw_bytes)


def decoder_roofline(pool, stride, work, raw_stride, sizes, raw_bytes, reps=20, codec="xw4") -> dict:
    """Blobs in pool slots 0..n-1 decoded into work slots 0..n-1 in one launch, timed with HIP events
    on the stream it runs on; algorithmic bytes = the blobs' bytes read + the packages' bytes written."""
    import torch

    from mixture_experts_layer_token_amd import api

    n = len(sizes)
    pairs = torch.tensor([[i, i] for i in range(n)], dtype=torch.int32, device="cuda")
    decode = api.moe_decompress_packages if codec == "xw4" else api.moe_decompress_rans
    for _ in range(3):
        decode(pool, stride, work, raw_stride, pairs, raw_bytes)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        decode(pool, stride, work, raw_stride, pairs, raw_bytes)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / reps
    alg = int(sum(sizes)) + n * raw_bytes
    kernel = "xw4_decode_kernel" if codec == "xw4" else "rns_decode_kernel"
    # (the rANS decoder is bound by each stream's serial chain of LDS lookups; its HBM fraction is
    # given for scale)
    return {"bound": "hbm" if codec == "xw4" else "latency", "kernel": "%s (%d packages per launch)" % (kernel, n),
            "achieved": round(alg / us / 1e3, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(alg / us / 1e3 / HBM_PEAK_GBS, 4), "traffic": None, "avg_launch_us": round(us, 2),
            "algorithmic_bytes_per_launch": alg, "timed_launches": reps}


def run_decoder(args):
    """A package decoder alone: 16 GLM-shaped experts encoded on the host (bf16 ones with the
    exponent-window code, 47 MB each; with --codec rans, INT4 ones with the rANS code, 12.6 MB each),
    their blobs decoded on the GPU in one launch per repetition; decoded bytes checked against the
    packages."""
    import numpy as np
    import torch

    from synth import workloads as W

    from mixture_experts_layer_token_amd import api
    from mixture_experts_layer_token_amd.layer import pack_bank

    codec = args.codec
    wfmt = "bf16" if codec == "xw4" else "int4g32"
    wl = W.WORKLOADS["glm"].with_(wfmt=wfmt, name="glm-" + wfmt)
    raw_bytes = api.moe_package_bytes(wl.H, wl.I, wfmt)
    n = 16
    host = pack_bank(wl, 0, list(range(n)), stride=raw_bytes)
    if codec == "xw4":
        blobs = [api.moe_compress_package(host[i]) for i in range(n)]
    else:
        split = api.package_split(wl.H, wl.I, wfmt)
        blobs = [api.moe_compress_rans(host[i], split) for i in range(n)]
    stride = (max(b.size for b in blobs) + 255) // 256 * 256
    pool = torch.zeros((n, stride), dtype=torch.uint8, device="cuda")
    for i, b in enumerate(blobs):
        pool[i, :b.size].copy_(torch.from_numpy(b))
    work = torch.empty((n, raw_bytes), dtype=torch.uint8, device="cuda")
    roof = decoder_roofline(pool, stride, work, raw_bytes, [b.size for b in blobs], raw_bytes, reps=args.steps,
                            codec=codec)
    ok = all(np.array_equal(work[i].cpu().numpy(), host[i]) for i in range(n))
    if not ok:
        raise RuntimeError("decoded packages differ from the originals")
    # one package per launch (what the expert cache's decode of a single miss costs)
    one = decoder_roofline(pool, stride, work, raw_bytes, [blobs[0].size], raw_bytes, reps=args.steps, codec=codec)
    roof["one_package_us"] = one["avg_launch_us"]
    us = roof["avg_launch_us"]
    return {"metric": "lossless package decode GB/s (blobs read + packages written)", "value": roof["achieved"],
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": 3, "ms_per_step": round(us / 1e3, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u8" if codec == "rans" else "bf16",
            "data": "synthetic (N(0,0.02) weights of GLM-shaped experts, %s)" % wfmt,
            "config": {"workload": "%s decode of %d glm-%s packages" % (codec, n, wfmt), "raw_bytes": raw_bytes,
                       "blob_bytes_mean": float(np.mean([b.size for b in blobs])),
                       "ratio": round(float(np.mean([b.size for b in blobs])) / raw_bytes, 5)},
            "roofline": roof, "decoded_equal": ok}



def offload_variant(model, wl, T, steps, xs, out, policy, period, overlap, pf, pin, belady):
    """One timed pass of `steps` decode steps through the model's layers with an empty cache of the
    given policy, prefetch heuristic and static pin; the run's figures."""
    import torch

    model.reset_cache(policy, period, overlap, prefetch=pf, pins=pin)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        for l in range(wl.layers):
            model.layer_forward(l, s, xs[(l, s)], out, time_copies=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    copy_s = model.copy_seconds()
    st = model.cache.stats()
    seen, cold = set(), 0
    per_epoch = {}
    for (s, l, n, h, m) in model.plans:
        a = per_epoch.setdefault(s // wl.rerank_every, [0, 0])
        a[0] += h
        a[1] += n
    # compulsory misses: first lookup of each (layer, expert) key
    for grp in model.groups:
        for key in grp:
            if key not in seen:
                seen.add(key)
                cold += 1
    name = policy if policy == "lru" else "%s/%d" % (policy, period)
    if pin is not None:
        name = "static-pin(%d/layer)+%s" % (len(pin[0]), name)
    bkey = (T, model.capacity)
    if bkey not in belady:
        belady[bkey] = belady_hits(model.capacity, model.groups)
    return {
        "T": T, "policy": name, "prefetch": pf or "none", "steps": steps,
        "ffn_of_hits_during_copies": overlap,
        "layers": wl.layers, "cache_slots": model.capacity, "wall_s": wall, "tokens_per_s": T * steps / wall,
        "hit_rate": st["hits"] / max(1, st["lookups"]),
        "hit_rate_cold_excluded": st["hits"] / max(1, st["lookups"] - cold),
        "hit_rate_per_epoch": [round(v[0] / max(1, v[1]), 4) for _, v in sorted(per_epoch.items())],
        "hit_rate_belady": belady[bkey] / max(1, st["lookups"]),
        "lookups": st["lookups"], "misses": st["misses"], "bytes_fetched": st["bytes_fetched"],
        "prefetch_fetches": st["prefetch_fetches"], "prefetch_hits": st["prefetch_hits"],
        "copy_busy_s": copy_s,
        "link_gbps_busy": st["bytes_fetched"] / max(1e-9, copy_s) / 1e9,
        "link_gbps_wall": st["bytes_fetched"] / wall / 1e9}


def run_offload(args):
    """256 decode steps through 8 layers whose experts live in pinned host memory (HBM cache)."""
    import torch

    from synth import workloads as W

    from mixture_experts_layer_token_amd import api
    from mixture_experts_layer_token_amd.layer import to_device_act
    from mixture_experts_layer_token_amd.offload import OffloadedModel

    wl = W.WORKLOADS["glm"]
    steps = min(args.offload_steps, wl.steps)
    Ts = [args.T] if args.T else [16, 1]
    model = OffloadedModel(wl, max(Ts), fill=False)
    rans = args.host_codec == "rans"
    if rans:
        # a second bank of rANS blobs of the same packages, in slots of the largest blob of a sample
        # plus 0.3% (the fill refuses any blob that does not fit), plain packages in the same HBM pool
        from mixture_experts_layer_token_amd.layer import pack_bank

        raw = model.raw_bytes
        sample = [pack_bank(wl, l, [e])[0, :raw] for l in range(wl.layers) for e in (0, 97)]
        largest = max(api.moe_compress_rans(p, model.split).size for p in sample)
        model_r = OffloadedModel(wl, max(Ts), capacity=model.capacity, fill=False, host_codec="rans",
                                 blob_bytes=(int(largest * 1.003) + 255) // 256 * 256)
    runs, belady = {}, {}
    for T in Ts:
        xs = {(l, s): to_device_act(W.activations(wl, T, l, s), wl.xdt) for s in range(steps) for l in range(wl.layers)}
        # route every (step, layer) once to know which experts the run touches; only those packages are
        # generated into the bank (the others are never fetched); the timed run routes again itself
        touched = {l: set() for l in range(wl.layers)}
        calib = {l: [] for l in range(wl.layers)}  # lookups of the first epoch: the static pin's profile
        ids = torch.empty((T, wl.k), dtype=torch.int32, device="cuda")
        gw = torch.empty((T, wl.k), dtype=torch.float32, device="cuda")
        for (l, s), x in xs.items():
            api.moe_route(x, model.wg[l], model.bias(l, s), wl.k, ids, gw)
            got = ids.cpu().numpy().ravel()
            touched[l] |= set(got.tolist())
            if s < wl.rerank_every:
                calib[l].append(got)
        for l in range(wl.layers):
            model.fill(l, touched[l] - model.filled.get(l, set()))
            model.filled[l] = model.filled.get(l, set()) | touched[l]
            if rans:  # the same packages, from the plain bank
                model_r.fill(l, touched[l] - model_r.filled.get(l, set()),
                             source=lambda l_, ids: np.stack([model.package(l_, e) for e in ids]))
                model_r.filled[l] = model_r.filled.get(l, set()) | touched[l]
        out = torch.empty((T, wl.H), dtype=torch.bfloat16, device="cuda")
        # half the slots pinned (the layers' most used experts over the first popularity epoch), LRU on the rest
        pins = static_pins(model, calib, model.capacity // 2 // wl.layers)
        if rans:  # both banks under the two policies, no prefetch
            variants = [(p, d, True, None, None) for p, d in POLICIES]
        else:
            variants = [(p, d, True, pf, None) for p, d in POLICIES for pf in PREFETCH]
            variants += [("lru", 0, True, None, pins)]
            if T == Ts[0]:  # the reported policy without the FFN/copy overlap
                variants.append((*POLICIES[-1], False, None, None))
        for bank, m in (("plain", model), ("rans", model_r if rans else None)):
            if m is None:
                continue
            m.reset_cache(prefetch=None)
            for l in range(wl.layers):  # warm the kernels through the full path (the cache is reset below)
                m.layer_forward(l, 0, xs[(l, 0)], out)
            for policy, period, overlap, pf, pin in variants:
                r = offload_variant(m, wl, T, steps, xs, out, policy, period, overlap, pf, pin, belady)
                r["bank"] = bank
                if bank == "rans":  # package bytes the blobs delivered per second of copy-stream time
                    r["packages_gbps_busy"] = r["misses"] * m.raw_bytes / max(1e-9, r["copy_busy_s"]) / 1e9
                runs[(T, bank, r["policy"], overlap, pf)] = r
                print("offload %s bank T=%d %s prefetch %s: %.1f tokens/s, hit %.4f" % (
                    bank, T, r["policy"], pf, r["tokens_per_s"], r["hit_rate"]), flush=True)
    head_bank = "rans" if rans else "plain"
    head = max((r for r in runs.values() if r["T"] == Ts[0] and r["ffn_of_hits_during_copies"]
                and r["bank"] == head_bank), key=lambda r: r["tokens_per_s"])
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
                   "cache_policy": head["policy"], "prefetch": head["prefetch"], "ffn_of_hits_during_copies": True,
                   "reported": "the fastest policy / prefetch combination at this T",
                   "bank": "rANS blobs (plain packages in HBM)" if rans else "plain packages",
                   "bank_bytes": wl.layers * wl.E * (model_r if rans else model).pkg_bytes},
        "roofline": {"bound": "link", "kernel": "hipMemcpyAsync host bank -> HBM slots (copy stream)",
                     "achieved": round(head["link_gbps_busy"], 2), "peak": PCIE_PEAK_GBS, "unit": "GB/s",
                     "frac": round(head["link_gbps_busy"] / PCIE_PEAK_GBS, 4), "traffic": None},
        "runs": [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()} for r in runs.values()],
    }
    if rans:
        plain = max((r for r in runs.values() if r["T"] == Ts[0] and r["bank"] == "plain"),
                    key=lambda r: r["tokens_per_s"])
        sizes = model_r.blob_sizes[model_r.blob_sizes > 0]
        out["vs_plain_bank"] = round(head["tokens_per_s"] / plain["tokens_per_s"], 4)
        out["compression"] = {"codec": "rans", "raw_bytes": model.raw_bytes, "blob_slot_bytes": model_r.pkg_bytes,
                              "ratio_mean": round(float(sizes.mean()) / model.raw_bytes, 5),
                              "ratio_max": round(float(sizes.max()) / model.raw_bytes, 5),
                              "experts": int(sizes.size)}
        n_dec = 16
        keys = [(l, e) for l in range(wl.layers) for e in range(wl.E) if model_r.blob_sizes[l, e] > 0][:n_dec]
        blob_stride = model_r.pkg_bytes
        pool = torch.zeros((len(keys), blob_stride), dtype=torch.uint8, device="cuda")
        for i, (l, e) in enumerate(keys):
            pool[i].copy_(torch.from_numpy(model_r.package(l, e).copy()))
        work = torch.empty((len(keys), model.raw_bytes), dtype=torch.uint8, device="cuda")
        out["decoder_roofline"] = decoder_roofline(pool, blob_stride, work, model.raw_bytes,
                                                   [int(model_r.blob_sizes[k]) for k in keys], model.raw_bytes,
                                                   codec="rans")
        model_r.close()
    model.close()
    return out



SPEC_ACCEPT = (0.5, 0.7, 0.9)  # per-position draft acceptance rates the report is given for


def expected_accepted(T: int, alpha: float) -> float:
    """Accepted tokens per verification block of T = depth + 1 positions when each draft position is
    accepted with probability alpha until the first rejection, plus the target's own token:
    1 + alpha + ... + alpha^(T-1)."""
    return sum(alpha ** i for i in range(T))


def run_spec(args):
    """Speculative verification: one request's block of T = depth + 1 positions through the GLM-shaped
    INT4 layer resident in HBM, T = 1 (ordinary decode) to 4.  Grouping by expert reads each expert
    of the block once (the union); a position-by-position pass would read k experts per position.
    Reported per T: time per block, distinct experts, expert bytes per block with and without reuse,
    and per accepted token at the acceptance rates SPEC_ACCEPT."""
    import torch

    from synth import workloads as W

    from mixture_experts_layer_token_amd import api
    from mixture_experts_layer_token_amd.layer import build_layer, to_device_act

    wl = W.WORKLOADS["glm"].with_(name="glm-spec-int4", layers=1, steps=1, rerank_every=0)
    pkg = api.moe_package_bytes(wl.H, wl.I, wl.wfmt)
    layer = build_layer(wl, 4)
    layers = layer_instances(layer, args.layers or 4)  # (4 x 3.4 GB: a step's experts are not in the MALL)
    rows = []
    for T in (1, 2, 3, 4):
        xs_host = [W.activations(wl, T, 0, 2000 + r) for r in range(args.batches)]
        xs = [to_device_act(a, wl.xdt) for a in xs_host]
        outs = [torch.empty_like(x) for x in xs]
        touched = touched_per_batch(layer, xs, wl.E)
        steps = args.steps
        total_ms, _, gu_ms, dn_ms, _ = measure(layers, xs, outs, steps, min(args.warmup, steps), trace=True)
        graph_ms = measure_graph(layers, xs, outs, steps, min(args.warmup, steps))
        union = float(np.mean(touched))
        row = {"T": T, "depth": T - 1, "ms_per_block": round(graph_ms, 5),
               "eager_ms_per_block": round(total_ms / steps, 5), "ffn_us": round(1e3 * float(np.mean(gu_ms) + np.mean(dn_ms)), 2),
               "distinct_experts": union, "expert_bytes_union": int(union * pkg),
               "expert_bytes_no_reuse": T * wl.k * pkg,
               "hbm_gbps_experts": round(union * pkg / (graph_ms * 1e-3) / 1e9, 1), "per_accept_rate": []}
        for a in SPEC_ACCEPT:
            acc = expected_accepted(T, a)
            row["per_accept_rate"].append({
                "alpha": a, "accepted_per_block": round(acc, 4),
                "expert_bytes_per_accepted": int(union * pkg / acc),
                "expert_bytes_per_accepted_no_reuse": int(T * wl.k * pkg / acc),
                "accepted_tokens_per_s": round(acc / (graph_ms * 1e-3), 1)})
        rows.append(row)
    base = rows[0]["ms_per_block"]
    head = rows[-1]
    best = next(r for r in head["per_accept_rate"] if r["alpha"] == 0.7)
    return {
        "metric": "MoE-layer accepted tokens/s of speculative verification (block of depth + 1 positions) "
                  "+ expert bytes per accepted token",
        "value": best["accepted_tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_block"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp16",
        "data": "synthetic (one request's positions routed independently; N(0,1) activations, N(0,0.02) weights "
                "quantized to int4g32; per-position acceptance rate assumed, not measured)",
        "config": {"workload": wl.name, "T": 4, "depth": 3, "hidden": wl.H, "experts": wl.E, "top_k": wl.k,
                   "inter": wl.I, "alpha_reported": 0.7, "launch": "hipGraph replay",
                   "layer_instances": len(layers), "input_batches": args.batches},
        "blocks": rows,
        "block_vs_decode_time": [round(r["ms_per_block"] / base, 3) for r in rows],
    }


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
    ap.add_argument("--workload", default="mixtral",
                    choices=["mixtral", "gptoss", "kimi", "glm", "glm-bf16", "spec", "decoder"])
    ap.add_argument("--host-codec", default="none", choices=["none", "rans"],
                    help="glm offload: also run a bank of rANS blobs (decoded into plain HBM slots) and report it")
    ap.add_argument("--codec", default="xw4", choices=["xw4", "rans"],
                    help="decoder workload: exponent-window code of bf16 packages, or rANS code of INT4 ones")
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
    ap.add_argument("--mode", default="auto", choices=["auto", "decode", "prefill", "decode_mx"],
                    help="moe_expert_ffn mode of the timed steps (decode_mx: MXFP4 on the block-scaled MFMA)")
    ap.add_argument("--no-prefill", dest="prefill", action="store_false",
                    help="default (Mixtral decode) run: leave out the Kimi-shaped prefill leg")
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
    if args.workload == "spec":
        print(json.dumps(run_spec(args)), flush=True)
        return
    if args.workload == "glm-bf16":
        out = run_offload_compressed(args)
    elif args.workload == "decoder":
        out = run_decoder(args)
    else:
        out = run_offload(args) if args.workload in OFFLOAD else run(args)
    if args.workload == "mixtral" and args.prefill:
        out["prefill"] = prefill_leg(args)
    print(json.dumps(out), flush=True)


def prefill_leg(args) -> dict:
    """The metric's prefill half beside the decode headline: the Kimi-K2-shaped INT4 layer with its
    shared expert at T = 8192, MFMA utilisation of the routed gate/up kernel, oracle on sampled tokens."""
    import copy
    import gc

    import torch

    gc.collect()
    torch.cuda.empty_cache()
    pa = copy.copy(args)
    pa.workload, pa.T, pa.sweep, pa.graph, pa.layers, pa.mode = "kimi", None, False, False, None, "auto"
    pre = run(pa)
    keep = ("metric", "value", "unit", "ms_per_step", "steps", "warmup", "dtype", "data", "config", "roofline",
            "expert_ffn", "step_tflops", "cpu_baseline")
    return {k: pre[k] for k in keep if k in pre}


if __name__ == "__main__":
    main()
