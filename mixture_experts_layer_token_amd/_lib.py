"""Loads libmoe.so (built in-tree by build.py) and declares its C signatures.

There is no fallback: if the library is missing or cannot be loaded, every
entry point raises.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
SO = os.path.join(HERE, "libmoe.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "moe.h")

c_int, c_size_t, vp, i32p, f32p = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p


class MoeExperts(ctypes.Structure):
    _fields_ = [("H", c_int), ("I", c_int), ("E", c_int), ("fmt", c_int), ("packages", vp),
                ("pkg_stride", c_size_t), ("slot_of_expert", vp), ("n_slots", c_int)]


# moe_copy_fn: int (*)(void* ctx, void* dst, const void* src, size_t bytes, void* stream)
COPY_FN = ctypes.CFUNCTYPE(c_int, vp, vp, vp, c_size_t, vp)


class MoeCacheDesc(ctypes.Structure):
    _fields_ = [("host_bank", vp), ("pkg_bytes", c_size_t), ("L", c_int), ("E", c_int), ("device_pool", vp),
                ("slot_stride", c_size_t), ("capacity", c_int), ("policy", c_int), ("decay_period", c_int),
                ("copy", COPY_FN), ("copy_ctx", vp)]


class MoeCachePlan(ctypes.Structure):
    _fields_ = [("layer", c_int), ("n_ids", c_int), ("n_hits", c_int), ("n_misses", c_int),
                ("miss_ids", ctypes.c_int32 * 1024), ("miss_slots", ctypes.c_int32 * 1024),
                ("slot_of_expert", ctypes.c_int32 * 1024)]


class MoeCacheStats(ctypes.Structure):
    _fields_ = [("lookups", ctypes.c_int64), ("hits", ctypes.c_int64), ("misses", ctypes.c_int64),
                ("evictions", ctypes.c_int64), ("bytes_fetched", ctypes.c_int64),
                ("prefetch_fetches", ctypes.c_int64), ("prefetch_hits", ctypes.c_int64)]


SIGNATURES = {
    "moe_last_error": ([], ctypes.c_char_p),
    "moe_route": ([vp, c_int, c_int, c_int, vp, f32p, c_int, c_int, i32p, f32p, f32p, vp, c_size_t, vp], c_int),
    "moe_route_workspace": ([c_int, c_int, c_int, c_int], c_size_t),
    "moe_permute_workspace": ([c_int, c_int, c_int], c_size_t),
    "moe_permute": ([i32p, c_int, c_int, c_int, i32p, i32p, i32p, i32p, vp, c_size_t, vp], c_int),
    "moe_route_permute_workspace": ([c_int, c_int, c_int, c_int, c_int], c_size_t),
    "moe_route_permute": ([vp, c_int, c_int, c_int, vp, f32p, c_int, c_int, i32p, f32p, f32p, i32p, i32p, i32p, i32p,
                           vp, c_size_t, vp], c_int),
    "moe_compress_bound": ([c_size_t], c_size_t),
    "moe_compress_package": ([vp, c_size_t, vp, c_size_t, ctypes.POINTER(c_size_t)], c_int),
    "moe_decompress_packages": ([vp, c_size_t, vp, c_size_t, i32p, c_int, c_size_t, vp], c_int),
    "moe_compress_rans_bound": ([c_size_t], c_size_t),
    "moe_compress_rans": ([vp, c_size_t, c_size_t, vp, c_size_t, ctypes.POINTER(c_size_t)], c_int),
    "moe_decompress_rans": ([vp, c_size_t, vp, c_size_t, i32p, c_int, c_size_t, vp], c_int),
    "moe_package_bytes": ([c_int, c_int, c_int], c_size_t),
    "moe_pack_expert": ([c_int, c_int, c_int, vp, vp, vp, vp, vp, vp, vp, c_size_t], c_int),
    "moe_dequant_expert": ([vp, c_int, c_int, c_int, f32p, vp], c_int),
    "moe_ffn_workspace": ([ctypes.POINTER(MoeExperts), c_int, c_int, c_int], c_size_t),
    "moe_expert_ffn": ([ctypes.POINTER(MoeExperts), vp, c_int, c_int, c_int, i32p, i32p, f32p, c_int, vp, c_size_t,
                        vp], c_int),
    "moe_expert_ffn_noalloc": ([ctypes.POINTER(MoeExperts), vp, c_int, c_int, c_int, i32p, i32p, f32p, c_int, vp],
                               c_int),
    "moe_ffn_trace_events": ([vp], c_int),
    "moe_combine": ([f32p, f32p, i32p, c_int, c_int, c_int, f32p, vp, c_int, vp], c_int),
    "moe_cache_create": ([ctypes.POINTER(MoeCacheDesc), ctypes.POINTER(vp)], c_int),
    "moe_cache_plan": ([vp, c_int, i32p, c_int, ctypes.POINTER(MoeCachePlan)], c_int),
    "moe_cache_prefetch": ([vp, c_int, i32p, c_int, ctypes.POINTER(MoeCachePlan)], c_int),
    "moe_cache_pin": ([vp, c_int, i32p, c_int, ctypes.POINTER(MoeCachePlan)], c_int),
    "moe_cache_fetch": ([vp, ctypes.POINTER(MoeCachePlan), i32p, vp, vp], c_int),
    "moe_cache_set_rans": ([vp, vp, c_size_t, c_int, c_size_t], c_int),
    "moe_cache_stats": ([vp, ctypes.POINTER(MoeCacheStats)], c_int),
    "moe_cache_destroy": ([vp], None),
}

_lib = None


def header_symbols() -> list[str]:
    """Function names declared in include/moe.h."""
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", txt)))


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(SO):
            from . import build as _build

            _build.build()
        L = ctypes.CDLL(SO)
        for name, (args, res) in SIGNATURES.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("moe status %d: %s" % (code, msg))
        self.code = code


def check(rc: int) -> None:
    if rc != 0:
        raise MoeError(rc, lib().moe_last_error().decode())
