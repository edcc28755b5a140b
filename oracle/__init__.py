"""CPU oracle for the routed-expert MoE layer -- TEST INFRASTRUCTURE ONLY.

ctypes wrapper over ``liboracle.so`` (plain fp64 C in ``oracle.c``).  Only the
tests, the package smoke check and the benchmark's CPU-baseline leg may import
this package.  It shares no code with the HIP library.

``rank_gap_inputs`` conditions router inputs: it redraws (from the seeded
generator) every activation row whose top-(k+1) logits are not separated by at
least ``gap``, so that top-k selection and order are unambiguous for any
implementation whose logit error is far below the gap.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

DT = {"f32": 0, "bf16": 1}
FMT = {"f32": 0, "bf16": 1, "mxfp4": 2, "int4g32": 3}


def build(force: bool = False) -> str:
    """Compile liboracle.so: gcc -O2, no fast-math, OpenMP."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
             os.path.join(_HERE, "oracle.c"), "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


class _Expert(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int), ("w", ctypes.c_void_p * 3), ("s", ctypes.c_void_p * 3)]


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_SO)
        i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        L.oracle_decode.argtypes = [i32, vp, vp, i64, i64, vp]
        L.oracle_decode_act.argtypes = [i32, vp, i64, vp]
        L.oracle_router_logits.argtypes = [i32, vp, vp, vp, i64, i64, i64, vp]
        L.oracle_topk_gates.argtypes = [vp, i64, i64, i32, vp, vp]
        L.oracle_permute.argtypes = [vp, i64, i32, i64, vp, vp, vp, vp]
        L.oracle_ffn.argtypes = [ctypes.POINTER(_Expert), i64, i64, vp, i64, vp]
        L.oracle_moe_layer.argtypes = [i32, vp, i64, i64, vp, vp, i64, i32, i64, ctypes.POINTER(_Expert),
                                       ctypes.POINTER(_Expert), i64, vp, i64, vp, vp, vp]
        L.oracle_moe_layer.restype = i32
        L.oracle_lru.argtypes = [i64, i64, vp, vp, vp, vp, vp, vp]
        L.oracle_lru.restype = i32
        L.oracle_lfu_decay.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp, vp]
        L.oracle_lfu_decay.restype = i32
        L.oracle_belady.argtypes = [i64, i64, vp, vp, vp, vp]
        L.oracle_belady.restype = i32
        L.oracle_cache_sim.argtypes = [i64, i32, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp]
        L.oracle_cache_sim.restype = i32
        L.oracle_xw4_bound.argtypes = [i64]
        L.oracle_xw4_bound.restype = i64
        L.oracle_xw4_encode.argtypes = [vp, i64, vp, i64]
        L.oracle_xw4_encode.restype = i64
        L.oracle_xw4_decode.argtypes = [vp, i64, vp, i64]
        L.oracle_xw4_decode.restype = i32
        L.oracle_rns_bound.argtypes = [i64]
        L.oracle_rns_bound.restype = i64
        L.oracle_rns_encode.argtypes = [vp, i64, i64, vp, i64]
        L.oracle_rns_encode.restype = i64
        L.oracle_rns_decode.argtypes = [vp, i64, vp, i64]
        L.oracle_rns_decode.restype = i32
        for f in ("oracle_decode", "oracle_decode_act", "oracle_router_logits", "oracle_topk_gates",
                  "oracle_permute", "oracle_ffn"):
            getattr(L, f).restype = None
        _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous numpy"
    return a.ctypes.data_as(ctypes.c_void_p)


def _expert(ex: dict) -> _Expert:
    s = _Expert()
    s.fmt = FMT[ex["fmt"]]
    for m in range(3):
        s.w[m] = _p(ex["w"][m])
        s.s[m] = _p(ex["s"][m]) if ex["s"][m] is not None else None
    return s


def decode(fmt: str, w: np.ndarray, s, rows: int, K: int) -> np.ndarray:
    """Exact fp64 value of every weight of a [rows, K] matrix in format fmt."""
    out = np.empty((rows, K), dtype=np.float64)
    lib().oracle_decode(FMT[fmt], _p(w), _p(s), rows, K, _p(out))
    return out


def decode_act(dt: str, x: np.ndarray) -> np.ndarray:
    out = np.empty(x.shape, dtype=np.float64)
    lib().oracle_decode_act(DT[dt], _p(x), x.size, _p(out))
    return out


def router_logits(dt: str, x: np.ndarray, wg: np.ndarray, bias) -> np.ndarray:
    T, H = x.shape
    E = wg.shape[0]
    out = np.empty((T, E), dtype=np.float64)
    lib().oracle_router_logits(DT[dt], _p(x), _p(wg), _p(bias), T, H, E, _p(out))
    return out


def topk_gates(logits: np.ndarray, k: int):
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    lib().oracle_topk_gates(_p(np.ascontiguousarray(logits)), T, E, k, _p(ids), _p(w))
    return ids, w


def permute(ids: np.ndarray, E: int):
    T, k = ids.shape
    n = T * k
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    perm = np.empty(max(n, 1), dtype=np.int32)
    inv = np.empty(max(n, 1), dtype=np.int32)
    lib().oracle_permute(_p(np.ascontiguousarray(ids, dtype=np.int32)), T, k, E, _p(counts), _p(offsets),
                         _p(perm), _p(inv))
    return counts, offsets, perm[:n], inv[:n]


def ffn(ex: dict, H: int, I: int, x: np.ndarray) -> np.ndarray:
    """SwiGLU FFN of one expert on fp64 rows x [n, H]."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    n = x.shape[0]
    y = np.empty((n, H), dtype=np.float64)
    e = _expert(ex)
    lib().oracle_ffn(ctypes.byref(e), H, I, _p(x), n, _p(y))
    return y


def moe_layer(dt: str, x: np.ndarray, wg: np.ndarray, bias, k: int, I: int, experts: list, shared=None,
              I_shared: int = 0, sample=None):
    """Layer output (fp64) for the sampled tokens, with their routing (ids, gate weights).

    ``experts`` is a list of E logical-weight dicts (entries for experts that no
    sampled token routes to may be None).
    """
    T, H = x.shape
    E = wg.shape[0]
    sample = np.arange(T, dtype=np.int64) if sample is None else np.ascontiguousarray(sample, dtype=np.int64)
    ns = len(sample)
    arr = (_Expert * E)()
    keep = []
    for e in range(E):
        if experts[e] is not None:
            arr[e] = _expert(experts[e])
            keep.append(experts[e])
    sh = _expert(shared) if shared is not None else None
    out = np.empty((ns, H), dtype=np.float64)
    ids = np.empty((ns, k), dtype=np.int32)
    w = np.empty((ns, k), dtype=np.float64)
    rc = lib().oracle_moe_layer(DT[dt], _p(x), T, H, _p(wg), _p(bias), E, k, I, arr,
                                ctypes.byref(sh) if sh is not None else None, I_shared,
                                _p(sample), ns, _p(out), _p(ids), _p(w))
    assert rc == 0
    return out, ids, w


def _groups(groups):
    off = np.zeros(len(groups) + 1, dtype=np.int64)
    for g, a in enumerate(groups):
        off[g + 1] = off[g] + len(a)
    keys = np.concatenate([np.asarray(a, dtype=np.int64) for a in groups]) if groups else np.zeros(0, np.int64)
    return off, np.ascontiguousarray(keys, dtype=np.int64)


def lru(capacity: int, groups):
    """LRU over groups of keys -> (hits[g], misses[g], victims per group (list of arrays))."""
    off, keys = _groups(groups)
    G = len(groups)
    hits = np.zeros(G, np.int64)
    misses = np.zeros(G, np.int64)
    victims = np.zeros(max(len(keys), 1), np.int64)
    nv = np.zeros(G, np.int64)
    rc = lib().oracle_lru(capacity, G, _p(off), _p(keys), _p(hits), _p(misses), _p(victims), _p(nv))
    if rc != 0:
        raise ValueError("a group holds more distinct keys than the capacity")
    vo = np.concatenate([[0], np.cumsum(nv)])
    return hits, misses, [victims[vo[g]:vo[g + 1]].copy() for g in range(G)]


def lfu_decay(capacity: int, period: int, groups):
    """Use counts with decay (+1024 per group a key appears in, halved every `period` groups);
    victim = smallest (count, last use, key) not in the group -> (hits[g], misses[g], victims)."""
    off, keys = _groups(groups)
    G = len(groups)
    hits = np.zeros(G, np.int64)
    misses = np.zeros(G, np.int64)
    victims = np.zeros(max(len(keys), 1), np.int64)
    nv = np.zeros(G, np.int64)
    rc = lib().oracle_lfu_decay(capacity, period, G, _p(off), _p(keys), _p(hits), _p(misses), _p(victims), _p(nv))
    if rc != 0:
        raise ValueError("a group holds more distinct keys than the capacity")
    vo = np.concatenate([[0], np.cumsum(nv)])
    return hits, misses, [victims[vo[g]:vo[g + 1]].copy() for g in range(G)]


CACHE_KINDS = {"demand": 0, "prefetch": 1, "pin": 2}


def cache_sim(capacity: int, policy: str, period: int, groups, kinds):
    """The cache with prefetch and pin groups (kinds: 'demand' | 'prefetch' | 'pin' per group;
    policy 'lru' | 'lfu_decay') -> (hits[g], misses[g], victims per group, prefetch_hits)."""
    off, keys = _groups(groups)
    G = len(groups)
    k = np.array([CACHE_KINDS[x] for x in kinds], dtype=np.int32)
    hits = np.zeros(G, np.int64)
    misses = np.zeros(G, np.int64)
    victims = np.zeros(max(len(keys), 1), np.int64)
    nv = np.zeros(G, np.int64)
    ph = np.zeros(1, np.int64)
    rc = lib().oracle_cache_sim(capacity, {"lru": 0, "lfu_decay": 1}[policy], period, G, _p(off), _p(keys), _p(k),
                                _p(hits), _p(misses), _p(victims), _p(nv), _p(ph))
    if rc != 0:
        raise ValueError("a demand or pin group does not fit the cache")
    vo = np.concatenate([[0], np.cumsum(nv)])
    return hits, misses, [victims[vo[g]:vo[g + 1]].copy() for g in range(G)], int(ph[0])


def belady(capacity: int, groups):
    off, keys = _groups(groups)
    G = len(groups)
    hits = np.zeros(G, np.int64)
    misses = np.zeros(G, np.int64)
    rc = lib().oracle_belady(capacity, G, _p(off), _p(keys), _p(hits), _p(misses))
    if rc != 0:
        raise ValueError("a group holds more distinct keys than the capacity")
    return hits, misses


def xw4_encode(raw: np.ndarray) -> np.ndarray:
    """Exponent-window code of a bf16 package (uint8 bytes, size a multiple of 1024) -> blob bytes."""
    raw = np.ascontiguousarray(raw).view(np.uint8).ravel()
    cap = int(lib().oracle_xw4_bound(raw.size))
    if cap < 0:
        raise ValueError("package size %d is not a multiple of 1024" % raw.size)
    out = np.zeros(cap, np.uint8)
    n = int(lib().oracle_xw4_encode(_p(raw), raw.size, _p(out), cap))
    if n < 0:
        raise ValueError("encode failed")
    return out[:n].copy()


def xw4_decode(blob: np.ndarray, raw_bytes: int) -> np.ndarray:
    """Blob -> the package's raw_bytes bytes (ValueError if the blob is malformed)."""
    blob = np.ascontiguousarray(blob).view(np.uint8).ravel()
    out = np.zeros(raw_bytes, np.uint8)
    if lib().oracle_xw4_decode(_p(blob), blob.size, _p(out), raw_bytes) != 0:
        raise ValueError("malformed blob")
    return out


def rns_encode(raw: np.ndarray, q: int) -> np.ndarray:
    """Order-0 rANS code of a package (uint8 bytes) cut at byte q into two regions -> blob bytes."""
    raw = np.ascontiguousarray(raw).view(np.uint8).ravel()
    cap = int(lib().oracle_rns_bound(raw.size))
    out = np.zeros(cap, np.uint8)
    n = int(lib().oracle_rns_encode(_p(raw), raw.size, q, _p(out), cap))
    if n < 0:
        raise ValueError("encode failed")
    return out[:n].copy()


def rns_decode(blob: np.ndarray, raw_bytes: int) -> np.ndarray:
    blob = np.ascontiguousarray(blob).view(np.uint8).ravel()
    out = np.zeros(raw_bytes, np.uint8)
    if lib().oracle_rns_decode(_p(blob), blob.size, _p(out), raw_bytes) != 0:
        raise ValueError("malformed blob")
    return out


def min_gap(logits: np.ndarray, k: int) -> np.ndarray:
    """Smallest difference between consecutive sorted logits among each row's top min(k+1, E)."""
    m = min(k + 1, logits.shape[1])
    top = -np.sort(-logits, axis=1)[:, :m]
    if m < 2:
        return np.full(logits.shape[0], np.inf)
    return np.min(top[:, :-1] - top[:, 1:], axis=1)


def rank_gap_inputs(wl, T: int, layer: int = 0, step: int = 0, gap: float = 1e-3, max_attempts: int = 64,
                    return_logits: bool = False):
    """x [T, H] from the generator, every row redrawn until its top-(k+1) logits differ by >= gap.

    Returns (x, attempts) where attempts[t] is the redraw index row t ended on, plus the final
    fp64 logits [T, E] when return_logits is set.
    """
    from synth import workloads as W

    wg = W.router_weights(wl, layer)
    bias = W.router_bias(wl, layer, step)
    attempts = np.zeros(T, dtype=np.int64)
    x = W.activations(wl, T, layer, step)
    logits = router_logits(wl.xdt, x, wg, bias)
    bad = np.nonzero(min_gap(logits, wl.k) < gap)[0]
    while len(bad):
        attempts[bad] += 1
        if attempts.max() > max_attempts:
            raise RuntimeError("rank-gap redraw did not converge")
        x[bad] = W.activation_rows(wl, layer, step, bad, attempts[bad])
        lg = router_logits(wl.xdt, np.ascontiguousarray(x[bad]), wg, bias)
        logits[bad] = lg
        bad = bad[min_gap(lg, wl.k) < gap]
    return (x, attempts, logits) if return_logits else (x, attempts)
