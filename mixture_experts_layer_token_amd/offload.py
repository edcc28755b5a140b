"""Decode through an expert bank that lives in page-locked host memory.

Expert weights stay on the host; an HBM pool of `capacity` package slots caches
the most recently used ones ("What expert offloading actually costs", section
"Inside expert paging": expert math stays on the GPU, weights stream in on
demand and are addressed through stable logical slots).  Per layer and step:

  route (compute stream) -> ids to the host -> moe_cache_plan (host policy) ->
  moe_cache_fetch (one hipMemcpyAsync per miss + the slot table, copy stream,
  event) -> permute -> grouped FFN over the experts that were already resident
  (their slots only; the misses' entries are -1) -> the compute stream waits for
  the event -> grouped FFN over the fetched experts -> combine.

The FFN of the hits runs while the misses stream in (with `overlap=False` the
whole FFN waits for the copies).

Layers run strictly in order.  A slot evicted by a plan is never in use: the
host waits for the router of the layer being planned, and every earlier FFN
precedes that router on the compute stream.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import api
from .layer import MoeLayer, to_device_act


class PinnedBuffer:
    """Page-locked host memory from hipHostMalloc, viewed as a numpy uint8 array."""

    def __init__(self, nbytes: int):
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipHostMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t, ctypes.c_uint]
        self._hip.hipHostFree.argtypes = [ctypes.c_void_p]
        p = ctypes.c_void_p()
        rc = self._hip.hipHostMalloc(ctypes.byref(p), ctypes.c_size_t(nbytes), 0)
        if rc != 0 or not p.value:
            raise MemoryError("hipHostMalloc(%d) failed with %d" % (nbytes, rc))
        self.ptr, self.nbytes = p.value, nbytes
        self.array = np.ctypeslib.as_array((ctypes.c_uint8 * nbytes).from_address(self.ptr))

    def data_ptr(self) -> int:
        return self.ptr

    def close(self):
        if self.ptr:
            self.array = None
            self._hip.hipHostFree(ctypes.c_void_p(self.ptr))
            self.ptr = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class OffloadedModel:
    """L MoE layers whose experts live in a pinned host bank, cached in an HBM slot pool."""

    def __init__(self, wl, max_T: int, capacity: int | None = None, device="cuda", fill=True, policy="lru",
                 decay_period=0, overlap=True):
        from synth import workloads as W

        self.wl = wl
        self.L, self.E, self.H, self.I, self.k = wl.layers, wl.E, wl.H, wl.I, wl.k
        self.pkg_bytes = api.moe_package_bytes(wl.H, wl.I, wl.wfmt)
        self.stride = (self.pkg_bytes + 255) // 256 * 256
        self.capacity = capacity or int(wl.cache_frac * wl.layers * wl.E)
        self.bank = PinnedBuffer(self.L * self.E * self.pkg_bytes)
        if fill:
            for l in range(self.L):
                self.fill(l, list(range(self.E)))
        self.pool = torch.empty((self.capacity, self.stride), dtype=torch.uint8, device=device)
        self.policy, self.decay_period = policy, decay_period
        self.cache = api.ExpertCache(self.bank, self.pkg_bytes, self.L, self.E, self.pool, self.stride,
                                     self.capacity, policy, decay_period)
        self.slot_tables = [torch.full((self.E,), -1, dtype=torch.int32, device=device) for _ in range(self.L)]
        # slot tables of the two FFN passes (hits only, misses only), staged from pinned host memory;
        # a layer's staging buffers are rewritten only after its previous copies ran (the host waits
        # for that layer's router first)
        self.overlap = overlap
        i32 = dict(dtype=torch.int32)
        self.pass_dev = [[torch.full((self.E,), -1, device=device, **i32) for _ in range(2)] for _ in range(self.L)]
        self.pass_host = [[torch.full((self.E,), -1, pin_memory=True, **i32) for _ in range(2)] for _ in range(self.L)]
        self.pass_desc = [[api.experts_desc(wl.H, wl.I, wl.E, wl.wfmt, self.pool, self.stride, t, self.capacity)
                           for t in pd] for pd in self.pass_dev]
        self.wg = [to_device_act(W.router_weights(wl, l), wl.xdt, device) for l in range(self.L)]
        self.bias_cache = {}
        self.layers = []
        for l in range(self.L):
            lay = MoeLayer(wl.H, wl.I, wl.E, wl.k, wl.wfmt, wl.xdt, self.wg[l], None, self.pool, self.stride,
                           max_T=max_T, slot_of_expert=self.slot_tables[l], device=device)
            self.layers.append(lay)
        self.copy_stream = torch.cuda.Stream(device=device)
        self.ids_host = torch.empty((max_T, wl.k), dtype=torch.int32, pin_memory=True)
        self.done = torch.cuda.Event()
        self.done.record(self.copy_stream)  # creates the HIP event the library records into
        self.routed = torch.cuda.Event()
        self.copy_t0 = torch.cuda.Event(enable_timing=True)
        self.copy_t1 = torch.cuda.Event(enable_timing=True)
        self.copy_ms = 0.0
        self.plans = []
        self.groups = []
        self.filled = {}

    def reset_cache(self, policy=None, decay_period=None, overlap=None):
        """Empty the HBM cache (a new planner, optionally with another policy) and the run records."""
        if overlap is not None:
            self.overlap = overlap
        if policy is not None:
            self.policy = policy
        if decay_period is not None:
            self.decay_period = decay_period
        self.cache.close()
        self.cache = api.ExpertCache(self.bank, self.pkg_bytes, self.L, self.E, self.pool, self.stride,
                                     self.capacity, self.policy, self.decay_period)
        for t in self.slot_tables:
            t.fill_(-1)
        self.plans, self.groups, self.copy_ms = [], [], 0.0

    def fill(self, l: int, experts):
        """Generate and pack experts of layer l into the host bank."""
        from .layer import pack_bank

        experts = sorted(experts)
        for i in range(0, len(experts), 64):
            ids = experts[i:i + 64]
            host = pack_bank(self.wl, l, ids, stride=self.pkg_bytes)
            for j, e in enumerate(ids):
                o = (l * self.E + e) * self.pkg_bytes
                self.bank.array[o:o + self.pkg_bytes] = host[j]

    def package(self, l: int, e: int) -> np.ndarray:
        o = (l * self.E + e) * self.pkg_bytes
        return self.bank.array[o:o + self.pkg_bytes]

    def bias(self, l: int, step: int):
        from synth import workloads as W

        epoch = step // self.wl.rerank_every if self.wl.rerank_every else 0
        key = (l, epoch)
        if key not in self.bias_cache:
            b = W.router_bias(self.wl, l, step)
            self.bias_cache[key] = torch.from_numpy(b).cuda() if b is not None else None
        return self.bias_cache[key]

    def layer_forward(self, l: int, step: int, x: torch.Tensor, out: torch.Tensor | None = None,
                      time_copies: bool = False) -> torch.Tensor:
        lay = self.layers[l]
        T, k = x.shape[0], self.k
        if out is None:
            out = torch.empty((T, self.H), dtype=x.dtype, device=x.device)
        ids, w = lay.topk_ids[:T], lay.topk_w[:T]
        api.moe_route(x, self.wg[l], self.bias(l, step), k, ids, w, ws=lay.rws)
        host_ids = self.ids_host[:T]
        host_ids.copy_(ids, non_blocking=True)
        self.routed.record()
        self.routed.synchronize()  # the router's choice, on the host
        hid = host_ids.numpy()
        plan = self.cache.plan(l, hid)
        self.plans.append((step, l, plan.n_ids, plan.n_hits, plan.n_misses))
        self.groups.append(set((l * self.E + hid.ravel()).tolist()))
        split = self.overlap and plan.n_hits > 0 and plan.n_misses > 0
        if split:
            table = np.ctypeslib.as_array(plan.slot_of_expert)[:self.E]
            miss = np.ctypeslib.as_array(plan.miss_ids)[:plan.n_misses]
            hit_t, miss_t = (h.numpy() for h in self.pass_host[l])
            hit_t[:] = table
            hit_t[miss] = -1
            miss_t[:] = -1
            miss_t[miss] = table[miss]
            for dev, host in zip(self.pass_dev[l], self.pass_host[l]):
                dev.copy_(host, non_blocking=True)
        if time_copies:
            self.copy_t0.record(self.copy_stream)
        self.cache.fetch(plan, self.slot_tables[l], self.copy_stream, self.done)
        if time_copies:
            self.copy_t1.record(self.copy_stream)
        if split:
            api.moe_permute(ids, self.E, lay.counts, lay.offsets, lay.perm_src[:T * k], lay.inv_perm[:T * k], lay.pws)
            api.moe_expert_ffn(self.pass_desc[l][0], x, k, lay.offsets, lay.perm_src, lay.y_perm, lay.ws)
            torch.cuda.current_stream().wait_event(self.done)
            api.moe_expert_ffn(self.pass_desc[l][1], x, k, lay.offsets, lay.perm_src, lay.y_perm, lay.ws)
        else:
            torch.cuda.current_stream().wait_event(self.done)
            api.moe_permute(ids, self.E, lay.counts, lay.offsets, lay.perm_src[:T * k], lay.inv_perm[:T * k], lay.pws)
            api.moe_expert_ffn(lay.desc, x, k, lay.offsets, lay.perm_src, lay.y_perm, lay.ws)
        api.moe_combine(lay.y_perm, w, lay.inv_perm, k, None, out)
        if time_copies:
            self.copy_t1.synchronize()
            self.copy_ms += self.copy_t0.elapsed_time(self.copy_t1)
        self.last_plan = plan
        return out

    def close(self):
        self.cache.close()
        self.bank.close()
