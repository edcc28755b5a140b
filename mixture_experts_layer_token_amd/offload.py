"""Decode through an expert bank that lives in page-locked host memory.

Expert weights stay on the host; an HBM pool of `capacity` package slots caches
the most recently used ones ("What expert offloading actually costs", section
"Inside expert paging": expert math stays on the GPU, weights stream in on
demand and are addressed through stable logical slots).  Per layer and step:

  route (compute stream) -> ids to the host -> moe_cache_plan (host policy) ->
  moe_cache_fetch (one hipMemcpyAsync per miss + the slot table, copy stream,
  event) -> [prefetch for the next layer: moe_cache_prefetch + its copies on the
  copy stream] -> permute -> grouped FFN over the experts that were already
  resident (their slots only; the misses' entries are -1) -> the compute stream
  waits for the event -> grouped FFN over the fetched experts -> combine.

The FFN of the hits runs while the misses stream in (with `overlap=False` the
whole FFN waits for the copies).  Fetching ahead needs no trained predictor
(the pages' related-abstracts list: an LRU cache, a static pin of popular
experts, experts fetched before they are needed): while layer l computes, the
next layer's experts of its previous step ("last") or its most used experts so
far ("popular") are prefetched; a static pin keeps each layer's most used
experts of a calibration window resident for the whole run.

Layers run strictly in order.  A slot evicted by a plan is never in use: the
host waits for the router of the layer being planned, and every earlier FFN
precedes that router on the compute stream; a prefetch never evicts the
experts of the layer just planned, whose FFN may still be running.

With `compressed=True` (bf16 experts) both tiers hold losslessly compressed
packages (the same page: compressed GPU memory beside host DRAM): the bank and
the HBM slots hold exponent-window blobs, so a miss moves about 3/4 of the
bytes and the same HBM holds more experts.  A layer's experts are decoded on
the compute stream into a small working pool of plain packages (`work_slots`,
shared by all layers), a group of at most that many at a time, each group
followed by its FFN pass: the hits' groups first, the misses' groups once
their copies landed.

With `host_codec="rans"` (meant for 4-bit experts, whose codes no fixed-width
code shrinks) only the host tier is compressed: the bank holds order-0 rANS
blobs, the HBM slots plain packages.  A miss copies its blob into a small
staging ring and the cache's decode stream writes the plain package into the
slot (moe_cache_set_rans), so the link carries fewer bytes, hits cost nothing
extra and the FFN reads the pool as in the plain case.
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
                 decay_period=0, overlap=True, prefetch=None, compressed=False, blob_bytes=None, work_slots=16,
                 host_codec=None, staging_slots=16):
        """`compressed`: bank and HBM slots hold blobs of `blob_bytes` bytes (a multiple of 256 that
        every expert's blob must fit; bf16 experts only), decoded through a working pool of
        `work_slots` plain packages.  `host_codec="rans"`: the bank holds rANS blobs in slots of
        `blob_bytes` bytes, decoded into the plain HBM slots as they arrive (through
        `staging_slots` device staging slots)."""
        from synth import workloads as W

        self.wl = wl
        self.L, self.E, self.H, self.I, self.k = wl.layers, wl.E, wl.H, wl.I, wl.k
        self.raw_bytes = api.moe_package_bytes(wl.H, wl.I, wl.wfmt)
        self.raw_stride = (self.raw_bytes + 255) // 256 * 256
        self.compressed = compressed
        self.host_codec = host_codec
        if host_codec not in (None, "rans") or (host_codec and compressed):
            raise ValueError("host_codec: None or 'rans' (not with compressed tiers)")
        if compressed or host_codec:
            if (compressed and wl.wfmt != "bf16") or not blob_bytes or blob_bytes % 256:
                raise ValueError("compressed banks hold blob slots of a multiple of 256 bytes (bf16 experts "
                                 "for compressed tiers)")
            self.pkg_bytes = blob_bytes  # bank stride; a miss copies at most one blob slot
        else:
            self.pkg_bytes = self.raw_bytes
        # pool slots: blobs (compressed tiers) or plain packages; the cache wants them >= the bank slot
        self.stride = (max(self.pkg_bytes, self.raw_bytes if host_codec else 0) + 255) // 256 * 256
        self.split = api.package_split(wl.H, wl.I, wl.wfmt)
        self.staging = (torch.empty((staging_slots, self.pkg_bytes), dtype=torch.uint8, device=device)
                        if host_codec else None)
        self.capacity = capacity or int(wl.cache_frac * wl.layers * wl.E)
        self.bank = PinnedBuffer(self.L * self.E * self.pkg_bytes)
        self.blob_sizes = np.zeros((self.L, self.E), np.int64)
        if fill:
            for l in range(self.L):
                self.fill(l, list(range(self.E)))
        self.pool = torch.empty((self.capacity, self.stride), dtype=torch.uint8, device=device)
        self.policy, self.decay_period = policy, decay_period
        self.cache = self._new_cache()
        self.slot_tables = [torch.full((self.E,), -1, dtype=torch.int32, device=device) for _ in range(self.L)]
        # slot tables of the two FFN passes (hits only, misses only), staged from pinned host memory;
        # a layer's staging buffers are rewritten only after its previous copies ran (the host waits
        # for that layer's router first)
        self.overlap = overlap
        i32 = dict(dtype=torch.int32)
        self.pass_dev = [[torch.full((self.E,), -1, device=device, **i32) for _ in range(2)] for _ in range(self.L)]
        self.pass_host = [[torch.full((self.E,), -1, pin_memory=True, **i32) for _ in range(2)] for _ in range(self.L)]
        if compressed:
            # decoded working pool of plain packages, shared by the layers
            self.n_work = min(self.E, max_T * self.k, work_slots)
            self.work = torch.empty((self.n_work, self.raw_stride), dtype=torch.uint8, device=device)
            # per layer, up to n_groups groups (the hits' and the misses' experts in groups of n_work):
            # a table over the working pool for the group's FFN pass and the decoder's pair list
            d_max = min(self.E, max_T * self.k)
            self.n_groups = (d_max + self.n_work - 1) // self.n_work + 1
            self.group_dev = [torch.full((self.n_groups, self.E), -1, device=device, **i32) for _ in range(self.L)]
            self.group_host = [torch.full((self.n_groups, self.E), -1, pin_memory=True, **i32) for _ in range(self.L)]
            self.pair_dev = [torch.full((self.n_groups, self.n_work, 2), -1, device=device, **i32)
                             for _ in range(self.L)]
            self.pair_host = [torch.full((self.n_groups, self.n_work, 2), -1, pin_memory=True, **i32)
                              for _ in range(self.L)]
            self.group_desc = [[api.experts_desc(wl.H, wl.I, wl.E, wl.wfmt, self.work, self.raw_stride, t, self.n_work)
                                for t in gd] for gd in self.group_dev]
            self.pass_desc = None
            self.last_group = []
        else:
            self.pass_desc = [[api.experts_desc(wl.H, wl.I, wl.E, wl.wfmt, self.pool, self.stride, t, self.capacity)
                               for t in pd] for pd in self.pass_dev]
        self.wg = [to_device_act(W.router_weights(wl, l), wl.xdt, device) for l in range(self.L)]
        self.bias_cache = {}
        self.layers = []
        for l in range(self.L):
            if compressed:  # the FFN reads the working pool through the group tables
                lay = MoeLayer(wl.H, wl.I, wl.E, wl.k, wl.wfmt, wl.xdt, self.wg[l], None, self.work, self.raw_stride,
                               max_T=max_T, slot_of_expert=self.group_dev[l][0], device=device)
            else:
                lay = MoeLayer(wl.H, wl.I, wl.E, wl.k, wl.wfmt, wl.xdt, self.wg[l], None, self.pool, self.stride,
                               max_T=max_T, slot_of_expert=self.slot_tables[l], device=device)
            self.layers.append(lay)
        self.copy_stream = torch.cuda.Stream(device=device)
        self.ids_host = torch.empty((max_T, wl.k), dtype=torch.int32, pin_memory=True)
        self.done = torch.cuda.Event()
        self.done.record(self.copy_stream)  # creates the HIP event the library records into
        self.routed = torch.cuda.Event()
        self.prefetch = prefetch
        self._ev_pool = []  # timing events of the copy stream, reused from run to run
        self.filled = {}
        self._reset_records()

    def _new_cache(self):
        c = api.ExpertCache(self.bank, self.pkg_bytes, self.L, self.E, self.pool, self.stride, self.capacity,
                            self.policy, self.decay_period)
        if self.host_codec:
            c.set_rans(self.staging, self.pkg_bytes, self.raw_bytes)
        return c

    def _reset_records(self):
        self.plans, self.groups, self.events, self._copy_windows = [], [], [], []
        self.prev_ids = [None] * self.L  # distinct experts of each layer's previous step
        self.use_counts = np.zeros((self.L, self.E), np.int64)  # demand uses of each expert so far

    def _timing_event(self, i):
        while len(self._ev_pool) <= i:
            self._ev_pool.append(torch.cuda.Event(enable_timing=True))
        return self._ev_pool[i]

    def copy_seconds(self) -> float:
        """Busy time of the copy stream over the run: the windows from before each layer's first copy
        to after its last (demand, prefetch), read once the run is over."""
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in self._copy_windows) / 1e3

    def reset_cache(self, policy=None, decay_period=None, overlap=None, prefetch="keep", pins=None, capacity=None):
        """Empty the HBM cache (a new planner, optionally with another policy, prefetch heuristic and
        static pin) and the run records.  `pins`: {layer: expert ids} pinned (and fetched) at once;
        `capacity`: slots the planner may use (at most the pool's)."""
        if capacity is not None:
            if capacity > self.pool.shape[0]:
                raise ValueError("capacity %d exceeds the pool's %d slots" % (capacity, self.pool.shape[0]))
            self.capacity = capacity
        if overlap is not None:
            self.overlap = overlap
        if policy is not None:
            self.policy = policy
        if decay_period is not None:
            self.decay_period = decay_period
        if prefetch != "keep":
            self.prefetch = prefetch
        self.copy_stream.synchronize()  # (the old cache's copies and decodes are over)
        self.cache.close()
        self.cache = self._new_cache()
        for t in self.slot_tables:
            t.fill_(-1)
        self._reset_records()
        for l, ids in sorted((pins or {}).items()):
            ids = np.asarray(sorted(set(int(e) for e in ids)), dtype=np.int32)
            plan = self.cache.pin(l, ids)
            self.events.append(("pin", l, ids))
            self.cache.fetch(plan, None, self.copy_stream)
        self.copy_stream.synchronize()

    def prefetch_candidates(self, l: int):
        """Experts of layer l to fetch ahead of its router, by the current heuristic."""
        prev = self.prev_ids[l]
        if self.prefetch is None or prev is None:
            return None
        if self.prefetch == "last":
            return prev
        if self.prefetch == "popular":  # as many as the layer touched last time, most used first
            order = np.argsort(-self.use_counts[l], kind="stable")
            return np.sort(order[:len(prev)]).astype(np.int32)
        raise ValueError("prefetch heuristic %r" % (self.prefetch,))

    def fill(self, l: int, experts, source=None):
        """Generate and pack experts of layer l into the host bank (compressed: their blobs).
        `source(l, ids)`: the packages ([len(ids), raw_bytes] uint8) in place of generating them."""
        import concurrent.futures as cf

        from .layer import _workers, pack_bank

        experts = sorted(experts)
        for i in range(0, len(experts), 64):
            ids = experts[i:i + 64]
            host = source(l, ids) if source else pack_bank(self.wl, l, ids, stride=self.raw_bytes)
            if not self.compressed and not self.host_codec:
                for j, e in enumerate(ids):
                    o = (l * self.E + e) * self.pkg_bytes
                    self.bank.array[o:o + self.pkg_bytes] = host[j]
                continue

            def one(j):
                e = ids[j]
                blob = (api.moe_compress_package(host[j]) if self.compressed
                        else api.moe_compress_rans(host[j], self.split))
                if blob.size > self.pkg_bytes:
                    raise ValueError("layer %d expert %d: blob of %d bytes exceeds the %d-byte slot"
                                     % (l, e, blob.size, self.pkg_bytes))
                o = (l * self.E + e) * self.pkg_bytes
                self.bank.array[o:o + blob.size] = blob
                self.bank.array[o + blob.size:o + self.pkg_bytes] = 0
                self.blob_sizes[l, e] = blob.size

            with cf.ThreadPoolExecutor(max_workers=_workers()) as pool:
                list(pool.map(one, range(len(ids))))

    def package(self, l: int, e: int) -> np.ndarray:
        """The bank's bytes of expert e of layer l (compressed: its blob slot)."""
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
        api.moe_route_permute(x, self.wg[l], self.bias(l, step), k, ids, w, lay.counts, lay.offsets,
                              lay.perm_src[:T * k], lay.inv_perm[:T * k], ws=lay.rws)
        host_ids = self.ids_host[:T]
        host_ids.copy_(ids, non_blocking=True)
        self.routed.record()
        self.routed.synchronize()  # the router's choice, on the host
        hid = host_ids.numpy()
        plan = self.cache.plan(l, hid)
        self.plans.append((step, l, plan.n_ids, plan.n_hits, plan.n_misses))
        self.groups.append(set((l * self.E + hid.ravel()).tolist()))
        distinct = np.unique(hid).astype(np.int32)
        self.events.append(("demand", l, distinct))
        self.prev_ids[l] = distinct
        self.use_counts[l][distinct] += 1
        split = self.overlap and plan.n_hits > 0 and plan.n_misses > 0
        if self.compressed:
            groups = self._stage_decode(l, plan, distinct)
        elif split:
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
            t0 = self._timing_event(2 * len(self._copy_windows))
            t0.record(self.copy_stream)
        self.cache.fetch(plan, self.slot_tables[l], self.copy_stream, self.done)
        # fetch ahead for the next layer: its copies queue behind this layer's on the copy stream (the
        # next layer's own fetch event covers them); this layer's FFN waits only for its own
        nl = (l + 1) % self.L
        cand = self.prefetch_candidates(nl)
        if cand is not None and len(cand):
            pf = self.cache.prefetch(nl, cand)
            self.events.append(("prefetch", nl, np.asarray(cand, np.int32)))
            if pf.n_misses:
                self.cache.fetch(pf, None, self.copy_stream)
        if time_copies:
            t1 = self._timing_event(2 * len(self._copy_windows) + 1)
            t1.record(self.copy_stream)
            self._copy_windows.append((t0, t1))
        if self.compressed:
            # each group: decode its experts into the working pool, then their FFN pass (the next
            # group's decode follows that FFN on the stream); the misses' groups after their copies
            # (all groups after them without the overlap)
            waited = False
            for j, (is_miss, n) in enumerate(groups):
                if not waited and (is_miss or not self.overlap):
                    torch.cuda.current_stream().wait_event(self.done)
                    waited = True
                api.moe_decompress_packages(self.pool, self.stride, self.work, self.raw_stride, self.pair_dev[l][j],
                                            self.raw_bytes, n=n)
                api.moe_expert_ffn(self.group_desc[l][j], x, k, lay.offsets, lay.perm_src, lay.y_perm, lay.ws)
            if not waited:
                torch.cuda.current_stream().wait_event(self.done)
        elif split:
            api.moe_expert_ffn(self.pass_desc[l][0], x, k, lay.offsets, lay.perm_src, lay.y_perm, lay.ws)
            torch.cuda.current_stream().wait_event(self.done)
            api.moe_expert_ffn(self.pass_desc[l][1], x, k, lay.offsets, lay.perm_src, lay.y_perm, lay.ws)
        else:
            torch.cuda.current_stream().wait_event(self.done)
            api.moe_expert_ffn(lay.desc, x, k, lay.offsets, lay.perm_src, lay.y_perm, lay.ws)
        api.moe_combine(lay.y_perm, w, lay.inv_perm, k, None, out)
        self.last_plan = plan
        return out

    def _stage_decode(self, l, plan, distinct):
        """Compressed tiers: the layer's experts in groups of at most n_work (the hits' first, then
        the misses'); per group, a table over the working pool (expert -> its rank in the group) and
        the decoder's (blob slot, pool slot) pairs, staged through pinned memory to the device on the
        compute stream.  Returns [(group of misses?, experts in it)]."""
        blob_slot = np.ctypeslib.as_array(plan.slot_of_expert)[:self.E]
        is_miss = np.zeros(self.E, bool)
        is_miss[np.ctypeslib.as_array(plan.miss_ids)[:plan.n_misses]] = True
        tables, pairs = self.group_host[l].numpy(), self.pair_host[l].numpy()
        tables[:] = -1
        groups = []
        for miss in (False, True):
            ids = distinct[is_miss[distinct] == miss]
            for g0 in range(0, len(ids), self.n_work):
                g = ids[g0:g0 + self.n_work]
                j = len(groups)
                tables[j, g] = np.arange(len(g), dtype=np.int32)
                pairs[j, :len(g), 0] = blob_slot[g]
                pairs[j, :len(g), 1] = np.arange(len(g), dtype=np.int32)
                groups.append((miss, len(g)))
                self.last_group = g.tolist()
        self.group_dev[l].copy_(self.group_host[l], non_blocking=True)
        self.pair_dev[l].copy_(self.pair_host[l], non_blocking=True)
        return groups

    def close(self):
        self.cache.close()
        self.bank.close()
