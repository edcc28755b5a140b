"""One routed-expert MoE layer on the device: weights, buffers and the four calls.

``MoeLayer.forward`` runs route -> permute -> grouped expert FFN (-> shared
expert) -> combine, each a libmoe.so call on the current stream, with all
intermediate buffers allocated once.  ``build_layer`` fills a layer from a
seeded synthetic workload (``synth.workloads``), packing each expert on the
host and copying the packages into one device bank.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np
import torch

from . import api


def to_device_act(a: np.ndarray, xdt: str, device="cuda") -> torch.Tensor:
    """Generator output (float32, or bf16 bits in uint16) -> device tensor of dtype xdt."""
    if xdt == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)


class MoeLayer:
    def __init__(self, H, I, E, k, fmt, xdt, w_router, bias, packages, pkg_stride, shared_packages=None,
                 max_T=1, slot_of_expert=None, device="cuda"):
        self.H, self.I, self.E, self.k, self.fmt, self.xdt = H, I, E, k, fmt, xdt
        self.w_router, self.bias = w_router, bias
        self.packages, self.pkg_stride = packages, pkg_stride
        self.slot_of_expert = slot_of_expert
        self.desc = api.experts_desc(H, I, E, fmt, packages, pkg_stride, slot_of_expert)
        self.shared = shared_packages
        if shared_packages is not None:
            self.shared_desc = api.experts_desc(H, I, 1, "bf16", shared_packages, shared_packages.shape[-1])
        self.device = device
        self._alloc(max_T)

    def set_slots(self, slot_of_expert):
        self.slot_of_expert = slot_of_expert
        self.desc = api.experts_desc(self.H, self.I, self.E, self.fmt, self.packages, self.pkg_stride,
                                     slot_of_expert)

    def _alloc(self, T):
        d, k, H, E = self.device, self.k, self.H, self.E
        self.max_T = T
        n = max(T * k, 1)
        i32 = dict(dtype=torch.int32, device=d)
        self.topk_ids = torch.empty((T, k), **i32)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=d)
        self.counts = torch.empty(E, **i32)
        self.offsets = torch.empty(E + 1, **i32)
        self.perm_src = torch.empty(n, **i32)
        self.inv_perm = torch.empty(n, **i32)
        self.y_perm = torch.empty((n, H), dtype=torch.float32, device=d)
        # the workspace serves every mode this layer's format has (MXFP4: also the block-scaled one)
        modes = ("auto", "decode", "prefill") + (("decode_mx",) if self.fmt == "mxfp4" else ())
        ws = max(api.moe_ffn_workspace(self.desc, T, k, m) for m in modes)
        if self.shared is not None:
            ws = max(ws, api.moe_ffn_workspace(self.shared_desc, T, 1))
            self.sh_offsets = torch.tensor([0, T], **i32)
            self.sh_perm = torch.arange(T, **i32)
            self.sh_y = torch.empty((T, H), dtype=torch.float32, device=d)
        self.ws = torch.empty(max(ws, 256), dtype=torch.uint8, device=d)
        # every batch size up to T may be routed and grouped with this buffer
        rws = max(api.moe_route_permute_workspace(t, H, E, k, self.xdt) for t in range(1, T + 1))
        self.rws = torch.empty(max(rws, 256), dtype=torch.uint8, device=d)

    def forward(self, x: torch.Tensor, out: torch.Tensor | None = None, mode="auto", trace=None) -> torch.Tensor:
        """One layer forward on the current stream.  `trace`: optional ctypes array of 3 HIP events
        recorded around the routed expert FFN's kernels (moe_ffn_trace_events)."""
        T = x.shape[0]
        if T > self.max_T:
            self._alloc(T)
        k = self.k
        if out is None:
            out = torch.empty((T, self.H), dtype=x.dtype, device=x.device)
        ids, w = self.topk_ids[:T], self.topk_w[:T]
        api.moe_route_permute(x, self.w_router, self.bias, k, ids, w, self.counts, self.offsets, self.perm_src[:T * k],
                              self.inv_perm[:T * k], ws=self.rws)
        if trace is not None:
            api.lib().moe_ffn_trace_events(trace)
        try:
            api.moe_expert_ffn(self.desc, x, k, self.offsets, self.perm_src, self.y_perm, self.ws, mode)
        finally:
            if trace is not None:
                api.lib().moe_ffn_trace_events(None)
        sh = None
        if self.shared is not None:
            if T != self.sh_perm.numel():
                self.sh_offsets = torch.tensor([0, T], dtype=torch.int32, device=x.device)
                self.sh_perm = torch.arange(T, dtype=torch.int32, device=x.device)
            api.moe_expert_ffn(self.shared_desc, x, 1, self.sh_offsets, self.sh_perm, self.sh_y, self.ws, mode)
            sh = self.sh_y[:T]
        api.moe_combine(self.y_perm, w, self.inv_perm, k, sh, out)
        return out


def _workers():
    return min(16, os.cpu_count() or 1)


def pack_bank(wl, layer: int, experts, fmt: str | None = None, stride: int | None = None,
              weights=None) -> np.ndarray:
    """Host [len(experts), stride] uint8 bank of packed experts of one layer (parallel over experts).
    `weights`: optional mapping expert -> logical weights already generated (else generated here)."""
    from synth import workloads as W

    fmt = fmt or wl.wfmt
    nb = api.moe_package_bytes(wl.H, wl.I, fmt)
    stride = stride or (nb + 255) // 256 * 256
    bank = np.zeros((len(experts), stride), dtype=np.uint8)

    def one(i):
        e = experts[i]
        ex = weights[e] if weights is not None else W.expert_weights(wl, layer, e)
        api.moe_pack_expert(wl.H, wl.I, fmt, ex, bank[i, :nb])

    with cf.ThreadPoolExecutor(max_workers=_workers()) as pool:
        list(pool.map(one, range(len(experts))))
    return bank


def build_layer(wl, max_T: int, layer: int = 0, step: int = 0, device="cuda", weights=None) -> MoeLayer:
    """Device layer for workload `wl` (layer index `layer`; router bias of `step`'s popularity epoch).
    `weights`: optional mapping expert -> logical weights already generated."""
    from synth import workloads as W

    nb = api.moe_package_bytes(wl.H, wl.I, wl.wfmt)
    stride = (nb + 255) // 256 * 256
    packages = torch.empty((wl.E, stride), dtype=torch.uint8, device=device)
    chunk = max(1, min(wl.E, (1 << 30) // stride))  # pack ~1 GiB at a time on the host
    for e0 in range(0, wl.E, chunk):
        ids = list(range(e0, min(wl.E, e0 + chunk)))
        host = pack_bank(wl, layer, ids, stride=stride, weights=weights)
        packages[e0:e0 + len(ids)].copy_(torch.from_numpy(host))
    wg = to_device_act(W.router_weights(wl, layer), wl.xdt, device)
    b = W.router_bias(wl, layer, step)
    bias = torch.from_numpy(b).to(device) if b is not None else None
    shared = None
    if wl.shared:
        sw = W.shared_weights(wl, layer)
        snb = api.moe_package_bytes(wl.H, wl.I, "bf16")
        sstride = (snb + 255) // 256 * 256
        host = np.zeros((1, sstride), dtype=np.uint8)
        api.moe_pack_expert(wl.H, wl.I, "bf16", sw, host[0, :snb])
        shared = torch.from_numpy(host).to(device)
    return MoeLayer(wl.H, wl.I, wl.E, wl.k, wl.wfmt, wl.xdt, wg, bias, packages, stride, shared, max_T=max_T,
                    device=device)
