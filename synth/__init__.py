"""Seeded synthetic inputs for the routed-expert MoE layer.

Thin ctypes wrapper over ``libsynth.so`` (built from ``synth.c`` next to this
file).  The module draws inputs only -- activations, router weights, per-expert
bias, expert weights in plain or block-quantized form -- and holds none of the
layer's arithmetic.  Both the HIP path and the CPU oracle consume its output.

Every tensor is addressed by a 64-bit stream id derived from a tuple of names
and indices (``stream_id``), so any expert of any layer can be regenerated on
its own at any time, on any machine, with the same bytes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile libsynth.so with gcc (host code only)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
             os.path.join(_HERE, "synth.c"), "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_SO)
        u64, i64, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        L.synth_stream_key.argtypes = [u64, u64]
        L.synth_stream_key.restype = u64
        L.synth_raw_u64.argtypes = [u64, u64, u64]
        L.synth_raw_u64.restype = u64
        L.synth_draw_key.argtypes = [u64, u64]
        L.synth_draw_key.restype = u64
        for name in ("synth_uniform_f64",):
            getattr(L, name).argtypes = [u64, u64, u64, i64, vp]
            getattr(L, name).restype = None
        for name in ("synth_normal_f64", "synth_normal_f32", "synth_normal_bf16"):
            getattr(L, name).argtypes = [u64, u64, u64, i64, dbl, vp]
            getattr(L, name).restype = None
        for name in ("synth_quant_mxfp4", "synth_quant_int4g32"):
            getattr(L, name).argtypes = [u64, u64, i64, i64, dbl, vp, vp]
            getattr(L, name).restype = None
        _lib = L
    return _lib


_FNV_OFF = 0xCBF29CE484222325
_FNV_PRIME = 0x100000001B3


def stream_id(*parts) -> int:
    """Stable 64-bit id of a tensor: FNV-1a over '/'-joined parts."""
    h = _FNV_OFF
    for b in "/".join(str(p) for p in parts).encode():
        h ^= b
        h = (h * _FNV_PRIME) & 0xFFFFFFFFFFFFFFFF
    return h


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def raw_u64(seed: int, stream: int, i: int) -> int:
    return int(lib().synth_raw_u64(seed, stream, i))


def uniform(seed: int, stream: int, n: int, offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    lib().synth_uniform_f64(seed, stream, offset, n, _ptr(out))
    return out


def normal(seed: int, stream: int, shape, sigma: float, dtype: str, offset: int = 0) -> np.ndarray:
    """N(0, sigma) samples. dtype 'f64' | 'f32' | 'bf16' (bf16 returned as uint16 bit patterns, RNE)."""
    n = int(np.prod(shape))
    if dtype == "f64":
        out = np.empty(n, dtype=np.float64)
        lib().synth_normal_f64(seed, stream, offset, n, sigma, _ptr(out))
    elif dtype == "f32":
        out = np.empty(n, dtype=np.float32)
        lib().synth_normal_f32(seed, stream, offset, n, sigma, _ptr(out))
    elif dtype == "bf16":
        out = np.empty(n, dtype=np.uint16)
        lib().synth_normal_bf16(seed, stream, offset, n, sigma, _ptr(out))
    else:
        raise ValueError(dtype)
    return out.reshape(shape)


def quant_mxfp4(seed: int, stream: int, rows: int, K: int, sigma: float):
    """N(0, sigma) [rows, K] quantized to MXFP4 -> (codes uint8 [rows, K/2], E8M0 scales uint8 [rows, K/32])."""
    assert K % 32 == 0
    codes = np.empty((rows, K // 2), dtype=np.uint8)
    scales = np.empty((rows, K // 32), dtype=np.uint8)
    lib().synth_quant_mxfp4(seed, stream, rows, K, sigma, _ptr(codes), _ptr(scales))
    return codes, scales


def quant_int4g32(seed: int, stream: int, rows: int, K: int, sigma: float):
    """N(0, sigma) [rows, K] quantized to INT4 group-32 -> (codes uint8 [rows, K/2], bf16 scales uint16 [rows, K/32])."""
    assert K % 32 == 0
    codes = np.empty((rows, K // 2), dtype=np.uint8)
    scales = np.empty((rows, K // 32), dtype=np.uint16)
    lib().synth_quant_int4g32(seed, stream, rows, K, sigma, _ptr(codes), _ptr(scales))
    return codes, scales


def permutation(seed: int, stream: int, n: int) -> np.ndarray:
    """Seeded Fisher-Yates shuffle of range(n)."""
    p = np.arange(n, dtype=np.int64)
    for i in range(n - 1, 0, -1):
        j = raw_u64(seed, stream, i) % (i + 1)
        p[i], p[j] = p[j], p[i]
    return p
