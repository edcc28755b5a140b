"""Python names for the C-ABI entry points of libmoe.so.

Each function marshals torch tensors (device memory) or numpy arrays (host
memory) into the pointers and sizes of the C call of the same name, on the
current torch stream unless one is given.  All computation happens in the
library's HIP kernels.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from ._lib import COPY_FN, MoeCacheDesc, MoeCachePlan, MoeCacheStats, MoeExperts, check, lib

FMT = {"f32": 0, "bf16": 1, "mxfp4": 2, "int4g32": 3}
DT = {"f32": 0, "bf16": 1}
MODE = {"auto": 0, "decode": 1, "prefill": 2, "decode_mx": 3}
POLICY = {"lru": 0, "lfu_decay": 1}
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _dp(t):
    """Device pointer of a tensor (None -> NULL)."""
    if t is None:
        return None
    assert t.is_cuda and t.is_contiguous(), "expected a contiguous device tensor"
    return ctypes.c_void_p(t.data_ptr())


def _hp(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DT["f32"]
    if t.dtype == torch.bfloat16:
        return DT["bf16"]
    raise TypeError("activations must be float32 or bfloat16, got %s" % t.dtype)


def moe_route_workspace(T, H, E, xdt) -> int:
    return int(lib().moe_route_workspace(T, H, E, DT[xdt]))


def moe_route(x, w_router, bias, k, topk_ids, topk_w, logits=None, ws=None, stream=None):
    """`ws`: device workspace of at least moe_route_workspace bytes (allocated here if None)."""
    T, H = x.shape
    E = w_router.shape[0]
    if ws is None:
        need = moe_route_workspace(T, H, E, "bf16" if x.dtype == torch.bfloat16 else "f32")
        ws = torch.empty(need, dtype=torch.uint8, device=x.device) if need else None
    check(lib().moe_route(_dp(x), _dt(x), T, H, _dp(w_router), _dp(bias), E, k, _dp(topk_ids), _dp(topk_w),
                          _dp(logits), _dp(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def moe_permute_workspace(T, k, E) -> int:
    return int(lib().moe_permute_workspace(T, k, E))


def moe_permute(topk_ids, E, counts, offsets, perm_src, inv_perm, ws=None, stream=None):
    """`ws`: device workspace of at least moe_permute_workspace bytes (allocated here if None)."""
    T, k = topk_ids.shape
    if ws is None:
        need = moe_permute_workspace(T, k, E)
        ws = torch.empty(need, dtype=torch.uint8, device=topk_ids.device) if need else None
    check(lib().moe_permute(_dp(topk_ids), T, k, E, _dp(counts), _dp(offsets), _dp(perm_src), _dp(inv_perm),
                            _dp(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def moe_route_permute_workspace(T, H, E, k, xdt) -> int:
    return int(lib().moe_route_permute_workspace(T, H, E, k, DT[xdt]))


def moe_route_permute(x, w_router, bias, k, topk_ids, topk_w, counts, offsets, perm_src, inv_perm, logits=None,
                      ws=None, stream=None):
    """moe_route then moe_permute in one call.  `ws`: device workspace of at least
    moe_route_permute_workspace bytes (allocated here if None)."""
    T, H = x.shape
    E = w_router.shape[0]
    if ws is None:
        need = moe_route_permute_workspace(T, H, E, k, "bf16" if x.dtype == torch.bfloat16 else "f32")
        ws = torch.empty(need, dtype=torch.uint8, device=x.device) if need else None
    check(lib().moe_route_permute(_dp(x), _dt(x), T, H, _dp(w_router), _dp(bias), E, k, _dp(topk_ids), _dp(topk_w),
                                  _dp(logits), _dp(counts), _dp(offsets), _dp(perm_src), _dp(inv_perm), _dp(ws),
                                  0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def moe_package_bytes(H, I, fmt) -> int:
    return int(lib().moe_package_bytes(H, I, FMT[fmt]))


def moe_pack_expert(H, I, fmt, ex: dict, out: np.ndarray | None = None) -> np.ndarray:
    """Pack one expert's logical weights (dict from synth.workloads.expert_weights) into a host package."""
    n = moe_package_bytes(H, I, fmt)
    if out is None:
        out = np.empty(n, dtype=np.uint8)
    w, s = ex["w"], ex["s"]
    check(lib().moe_pack_expert(H, I, FMT[fmt], _hp(w[0]), _hp(s[0]), _hp(w[1]), _hp(s[1]), _hp(w[2]), _hp(s[2]),
                                _hp(out), out.nbytes))
    return out


def moe_compress_bound(raw_bytes: int) -> int:
    return int(lib().moe_compress_bound(raw_bytes))


def moe_compress_package(raw: np.ndarray, out: np.ndarray | None = None) -> np.ndarray:
    """Lossless exponent-window code of one bf16 package (host bytes) -> its blob (a view of `out`)."""
    raw = np.ascontiguousarray(raw).view(np.uint8).ravel()
    cap = moe_compress_bound(raw.size)
    if out is None:
        out = np.empty(max(cap, 1), dtype=np.uint8)
    n = ctypes.c_size_t(0)
    check(lib().moe_compress_package(_hp(raw), raw.size, _hp(out), out.nbytes, ctypes.byref(n)))
    return out[:n.value]


def moe_decompress_packages(src, src_stride, dst, dst_stride, pairs, raw_bytes, n=None, stream=None):
    """Decode blobs into packages on the device: `pairs` is a device int32 [n, 2] tensor of
    (source slot, destination slot); `src` and `dst` are device tensors holding the slots."""
    n = pairs.shape[0] if n is None else n
    check(lib().moe_decompress_packages(_dp(src), src_stride, _dp(dst), dst_stride, _dp(pairs), n, raw_bytes,
                                        _stream(stream)))


def moe_compress_rans_bound(raw_bytes: int) -> int:
    return int(lib().moe_compress_rans_bound(raw_bytes))


def moe_compress_rans(raw: np.ndarray, split: int, out: np.ndarray | None = None) -> np.ndarray:
    """Order-0 rANS code of one package (host bytes, cut into regions at byte `split`) -> its blob."""
    raw = np.ascontiguousarray(raw).view(np.uint8).ravel()
    cap = int(lib().moe_compress_rans_bound(raw.size))
    if out is None:
        out = np.empty(cap, dtype=np.uint8)
    n = ctypes.c_size_t(0)
    check(lib().moe_compress_rans(_hp(raw), raw.size, split, _hp(out), out.nbytes, ctypes.byref(n)))
    return out[:n.value]


def moe_decompress_rans(src, src_stride, dst, dst_stride, pairs, raw_bytes, n=None, stream=None):
    n = pairs.shape[0] if n is None else n
    check(lib().moe_decompress_rans(_dp(src), src_stride, _dp(dst), dst_stride, _dp(pairs), n, raw_bytes,
                                    _stream(stream)))


def package_split(H, I, fmt) -> int:
    """Bytes of a package's first region for the rANS code: its weight codes (4-bit formats), all
    of it otherwise."""
    nb = moe_package_bytes(H, I, fmt)
    return 3 * H * I // 2 if fmt in ("mxfp4", "int4g32") else nb


def moe_dequant_expert(package, H, I, fmt, out, stream=None):
    check(lib().moe_dequant_expert(_dp(package), H, I, FMT[fmt], _dp(out), _stream(stream)))


def experts_desc(H, I, E, fmt, packages, pkg_stride, slot_of_expert=None, n_slots=None) -> MoeExperts:
    """`packages`: device tensor of packages, `pkg_stride` bytes apart (its leading dimension is the
    number of slots when a slot table is given)."""
    d = MoeExperts()
    d.H, d.I, d.E, d.fmt = H, I, E, FMT[fmt]
    d.packages = packages.data_ptr() if packages is not None else None
    d.pkg_stride = pkg_stride
    d.slot_of_expert = slot_of_expert.data_ptr() if slot_of_expert is not None else None
    if n_slots is None:
        n_slots = packages.numel() * packages.element_size() // pkg_stride if packages is not None else E
    d.n_slots = n_slots
    return d


def moe_ffn_workspace(desc: MoeExperts, T, k, mode="auto") -> int:
    return int(lib().moe_ffn_workspace(ctypes.byref(desc), T, k, MODE[mode]))


def moe_expert_ffn(desc: MoeExperts, x, k, offsets, perm_src, y_perm, ws, mode="auto", stream=None):
    T = x.shape[0]
    check(lib().moe_expert_ffn(ctypes.byref(desc), _dp(x), _dt(x), T, k, _dp(offsets), _dp(perm_src), _dp(y_perm),
                               MODE[mode], _dp(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                               _stream(stream)))


def moe_expert_ffn_noalloc(desc: MoeExperts, x, k, offsets, perm_src, y_perm, mode="auto", stream=None):
    """moe_expert_ffn with the library's static per-device scratch as workspace (no allocation)."""
    T = x.shape[0]
    check(lib().moe_expert_ffn_noalloc(ctypes.byref(desc), _dp(x), _dt(x), T, k, _dp(offsets), _dp(perm_src),
                                       _dp(y_perm), MODE[mode], _stream(stream)))


def moe_combine(y_perm, topk_w, inv_perm, k, shared_y, out, stream=None):
    T, H = out.shape
    check(lib().moe_combine(_dp(y_perm), _dp(topk_w), _dp(inv_perm), T, k, H, _dp(shared_y), _dp(out), _dt(out),
                            _stream(stream)))


class ExpertCache:
    """Owner of a moe_cache_t.  `bank` (pinned host tensor) and `pool` (device tensor) must outlive it."""

    def __init__(self, bank, pkg_bytes, L, E, pool, slot_stride, capacity, policy="lru", decay_period=0,
                 copy=None, bank_ptr=None, pool_ptr=None):
        """`copy`: optional copy engine, a Python callable (dst, src, bytes, stream) -> int (0 = ok);
        `bank_ptr` / `pool_ptr` then give the raw addresses it works on."""
        d = MoeCacheDesc()
        d.host_bank = bank_ptr if bank_ptr is not None else (bank.data_ptr() if bank is not None else None)
        d.pkg_bytes, d.L, d.E = pkg_bytes, L, E
        d.device_pool = pool_ptr if pool_ptr is not None else (pool.data_ptr() if pool is not None else None)
        d.slot_stride, d.capacity = slot_stride, capacity
        d.policy = POLICY[policy]
        d.decay_period = decay_period
        self._copy = None
        if copy is not None:
            self._copy = COPY_FN(lambda ctx, dst, src, n, stream: int(copy(dst, src, n, stream)))
            d.copy = self._copy
        self._keep = (bank, pool)
        h = ctypes.c_void_p()
        check(lib().moe_cache_create(ctypes.byref(d), ctypes.byref(h)))
        self.h = h
        self.E = E

    def set_rans(self, staging, staging_stride: int, raw_bytes: int):
        """The bank holds rANS blobs of raw_bytes packages; `staging` (device uint8 [slots, stride])
        takes each fetched blob before the cache's decode stream decodes it into its pool slot."""
        check(lib().moe_cache_set_rans(self.h, _dp(staging), staging_stride, staging.shape[0], raw_bytes))
        self._keep = self._keep + (staging,)

    def plan(self, layer, host_ids: np.ndarray) -> MoeCachePlan:
        ids = np.ascontiguousarray(host_ids, dtype=np.int32).ravel()
        p = MoeCachePlan()
        check(lib().moe_cache_plan(self.h, layer, _hp(ids), ids.size, ctypes.byref(p)))
        return p

    def prefetch(self, layer, host_ids: np.ndarray) -> MoeCachePlan:
        ids = np.ascontiguousarray(host_ids, dtype=np.int32).ravel()
        p = MoeCachePlan()
        check(lib().moe_cache_prefetch(self.h, layer, _hp(ids), ids.size, ctypes.byref(p)))
        return p

    def pin(self, layer, host_ids: np.ndarray) -> MoeCachePlan:
        ids = np.ascontiguousarray(host_ids, dtype=np.int32).ravel()
        p = MoeCachePlan()
        check(lib().moe_cache_pin(self.h, layer, _hp(ids), ids.size, ctypes.byref(p)))
        return p

    def fetch(self, plan: MoeCachePlan, dev_slot_of_expert, copy_stream, done_event=None):
        """`dev_slot_of_expert`: device tensor (or, with a copy engine, a raw address or None)."""
        ev = ctypes.c_void_p(done_event.cuda_event) if done_event is not None else None
        table = (ctypes.c_void_p(dev_slot_of_expert) if isinstance(dev_slot_of_expert, int)
                 else _dp(dev_slot_of_expert))
        stream = ctypes.c_void_p(copy_stream.cuda_stream) if copy_stream is not None else None
        check(lib().moe_cache_fetch(self.h, ctypes.byref(plan), table, stream, ev))

    def stats(self) -> dict:
        s = MoeCacheStats()
        check(lib().moe_cache_stats(self.h, ctypes.byref(s)))
        return {f: getattr(s, f) for f, _ in MoeCacheStats._fields_}

    def close(self):
        if self.h:
            lib().moe_cache_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
