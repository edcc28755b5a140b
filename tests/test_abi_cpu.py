"""Host-side checks of libmoe.so that need no GPU: exports, argument validation,
package sizes and the packer, and the LRU cache planner against the oracle."""
import ctypes

import numpy as np
import pytest

import oracle
from synth import workloads as W

import mixture_experts_layer_token_amd as moe
from mixture_experts_layer_token_amd import _lib
from mixture_experts_layer_token_amd.api import ExpertCache

L = moe.lib()
OK, INVALID, UNSUPPORTED, CAPACITY, WORKSPACE = 0, -1, -2, -4, -6


def test_every_header_symbol_is_exported():
    syms = moe.header_symbols()
    assert len(syms) >= 15
    for s in syms:
        assert hasattr(L, s), s
    assert set(_lib.SIGNATURES) == set(syms)


def test_route_workspace_sizes():
    # large bf16 batches: the router matrix repacked for the MFMA tile kernel + [T][E] fp32 logits
    # + offsets + the tile kernel's plan (at most 1 + ceil(T / 16) entries of 16 bytes) + its work counters
    plan = (1 + (8192 + 15) // 16) * 16
    assert moe.api.moe_route_workspace(8192, 7168, 384, "bf16") == (384 * 7168 * 2 + 8192 * 384 * 4 + 256
                                                                     + (plan + 255) // 256 * 256 + 256)
    # T * E <= 2^20: split over workgroups, KS ranges of partial logits (here KS = 1)
    assert moe.api.moe_route_workspace(300, 64, 24, "bf16") == 300 * 24 * 4
    assert moe.api.moe_route_workspace(50000, 64, 24, "bf16") == 0  # large, E not a multiple of 16: one kernel
    assert moe.api.moe_route_workspace(1, 2880, 128, "bf16") > 0
    assert moe.api.moe_route_workspace(16, 256, 8, "f32") == 0


def test_route_validation():
    # no pointer is touched before validation fails
    assert L.moe_route(None, 1, 4, 64, None, None, 0, 1, None, None, None, None, 0, None) == INVALID
    assert b"E=0" in L.moe_last_error()
    assert L.moe_route(None, 1, 4, 64, None, None, 8, 9, None, None, None, None, 0, None) == INVALID
    assert L.moe_route(None, 1, 4, 64, None, None, 64, 17, None, None, None, None, 0, None) == INVALID
    assert L.moe_route(None, 7, 4, 64, None, None, 8, 2, None, None, None, None, 0, None) == INVALID
    assert L.moe_route(None, 1, 4, 64, None, None, 8, 2, None, None, None, None, 0, None) == INVALID  # null x
    assert L.moe_route(None, 1, 0, 64, None, None, 8, 2, None, None, None, None, 0, None) == OK  # T = 0: nothing to do


def test_permute_workspace_sizes():
    assert moe.api.moe_permute_workspace(64, 2, 8) == 0  # one workgroup
    assert moe.api.moe_permute_workspace(1024, 8, 384) == 0
    assert moe.api.moe_permute_workspace(8192, 8, 384) == 8 * 32 * 384  # 32 blocks of 2048 indices
    assert moe.api.moe_permute_workspace(1025, 8, 16) == 8 * 5 * 16


def test_route_permute_workspace_sizes():
    al = lambda b: (b + 255) // 256 * 256
    # decode batches in bf16: only the router's partial logits (the single workgroup needs none)
    for T, H, E, k in ((1, 2880, 128, 4), (16, 7168, 384, 8), (16, 4096, 8, 2), (3, 64, 24, 2)):
        assert moe.api.moe_route_permute_workspace(T, H, E, k, "bf16") == al(moe.api.moe_route_workspace(T, H, E, "bf16"))
    # larger batches (T > 16), fp32, or H not a multiple of 32: route then permute
    for T, H, E, k, dt in ((17, 2880, 128, 4, "bf16"), (8192, 7168, 384, 8, "bf16"), (64, 4096, 64, 16, "bf16"),
                           (16, 256, 8, 2, "f32"), (4, 48, 8, 2, "bf16")):
        want = al(moe.api.moe_route_workspace(T, H, E, dt)) + al(moe.api.moe_permute_workspace(T, k, E))
        assert moe.api.moe_route_permute_workspace(T, H, E, k, dt) == want, (T, H, E, k, dt)
    assert moe.api.moe_route_permute_workspace(4, 64, 0, 2, "bf16") == 0


def test_route_permute_validation():
    n = [None] * 8
    assert L.moe_route_permute(None, 1, 4, 64, None, None, 0, 1, *n, 0, None) == INVALID
    assert b"E=0" in L.moe_last_error()
    assert L.moe_route_permute(None, 1, 4, 64, None, None, 8, 9, *n, 0, None) == INVALID  # k > E
    assert L.moe_route_permute(None, 1, 4, 64, None, None, 64, 17, *n, 0, None) == INVALID  # k > 16
    assert L.moe_route_permute(None, 7, 4, 64, None, None, 8, 2, *n, 0, None) == INVALID  # dtype
    assert L.moe_route_permute(None, 1, 4, 64, None, None, 8, 2, *n, 0, None) == INVALID  # null counts
    assert b"counts" in L.moe_last_error()
    assert L.moe_route_permute(None, 1, -1, 64, None, None, 8, 2, *n, 0, None) == INVALID


def test_permute_and_combine_validation():
    assert L.moe_permute(None, 4, 2, 0, None, None, None, None, None, 0, None) == INVALID
    assert L.moe_permute(None, 4, 0, 8, None, None, None, None, None, 0, None) == INVALID
    assert L.moe_permute(None, 4, 2, 8, None, None, None, None, None, 0, None) == INVALID
    assert L.moe_combine(None, None, None, 4, 2, 64, None, None, 5, None) == INVALID
    assert L.moe_combine(None, None, None, 4, 17, 64, None, None, 1, None) == INVALID
    assert L.moe_combine(None, None, None, 0, 2, 64, None, None, 1, None) == OK


def test_ffn_validation():
    d = moe.experts_desc(4096, 14336, 8, "bf16", None, moe.moe_package_bytes(4096, 14336, "bf16"))
    ref = ctypes.byref(d)
    assert L.moe_expert_ffn(ref, None, 1, 4, 2, None, None, None, 0, None, 0, None) == INVALID  # null pointers
    d.pkg_stride = 100
    assert L.moe_expert_ffn(ref, None, 1, 4, 2, None, None, None, 0, None, 0, None) == INVALID
    d2 = moe.experts_desc(100, 14336, 8, "bf16", None, 1 << 30)
    assert L.moe_expert_ffn(ctypes.byref(d2), None, 1, 4, 2, None, None, None, 0, None, 0, None) == UNSUPPORTED
    d3 = moe.experts_desc(4096, 14336, 0, "bf16", None, 1 << 30)
    assert L.moe_expert_ffn(ctypes.byref(d3), None, 1, 4, 2, None, None, None, 0, None, 0, None) == INVALID
    # workspace of bf16 experts, T = 64, k = 2 (128 pairs): the activation cast sized for fp32 input
    # (64 x 4096 bf16), h (128 x 14336 bf16), the streaming row-tile plan (1 + 128 / 16 + min(128, 8)
    # int4 entries) and the tile plan (1 + 0 + 8 entries) plus its 256 bytes of work counters, each
    # region rounded up to 256 bytes
    al = lambda b: (b + 255) // 256 * 256
    want = al(64 * 4096 * 2) + al(128 * 14336 * 2) + al((1 + 8 + 8) * 16) + al((1 + 0 + 8) * 16) + 256
    assert L.moe_ffn_workspace(ref, 64, 2, 0) == want


@pytest.mark.parametrize("fmt,H,I,want", [("bf16", 4096, 14336, 352321536), ("mxfp4", 2880, 2880, 13219200),
                                          ("int4g32", 7168, 2048, 24772608), ("int4g32", 5120, 1536, 13271040),
                                          ("f32", 256, 512, 1572864), ("bf16", 100, 64, 0)])
def test_package_bytes(fmt, H, I, want):
    assert moe.moe_package_bytes(H, I, fmt) == want


@pytest.mark.parametrize("fmt", ["f32", "bf16", "mxfp4", "int4g32"])
def test_packer_is_a_rearrangement(fmt):
    """Every code byte / element lands in the package exactly once (multiset of values preserved)."""
    wl = W.Workload(name="pk-" + fmt, H=224, E=2, k=1, I=352, wfmt=fmt, xdt="bf16", Ts=(1,), seed=9)
    ex = W.expert_weights(wl, 0, 1)
    pkg = moe.moe_pack_expert(wl.H, wl.I, fmt, ex)
    n = 3 * wl.H * wl.I
    if fmt in ("f32", "bf16"):
        dt = np.float32 if fmt == "f32" else np.uint16
        got = np.sort(pkg.view(dt))
        want = np.sort(np.concatenate([a.ravel() for a in ex["w"]]).view(dt))
        assert np.array_equal(got, want)
    else:
        codes = pkg[: n // 2]
        nib = np.concatenate([codes & 15, codes >> 4])
        src = np.concatenate([a.ravel() for a in ex["w"]])
        srcn = np.concatenate([src & 15, src >> 4])
        if fmt == "int4g32":
            srcn = (srcn + 8) & 15  # stored as q + 8
        assert np.array_equal(np.bincount(nib, minlength=16), np.bincount(srcn, minlength=16))
        assert pkg.size == n // 2 + (n // 32) * (1 if fmt == "mxfp4" else 2)


def test_pack_rejects_int4_scale_outside_binary16():
    H = I = 32
    codes = np.zeros((I, H // 2), np.uint8)
    s = np.full((I, 1), 0x3F80, np.uint16)  # 1.0
    s_bad = s.copy()
    s_bad[3, 0] = 0x4780 + 0x0100  # 2^16 * 1.x > 65504
    ex = {"w": [codes, codes, codes], "s": [s, s_bad, s]}
    with pytest.raises(moe.MoeError) as e:
        moe.moe_pack_expert(H, I, "int4g32", ex)
    assert e.value.code == UNSUPPORTED


# ------------------------------------------------------------------ cache planner (host only)

def _planner(cap, L_, E, policy="lru", period=0):
    return ExpertCache(None, 1 << 20, L_, E, None, 0, cap, policy, period)


@pytest.mark.parametrize("policy,period", [("lru", 0), ("lfu_decay", 32), ("lfu_decay", 0), ("lfu_decay", 1)])
def test_cache_planner_matches_oracle(policy, period):
    L_, E, cap, steps = 4, 64, 64, 120
    rng = np.random.default_rng(11)
    c = _planner(cap, L_, E, policy, period)
    groups, plans = [], []
    p = 1.0 / np.arange(1, E + 1) ** 1.2
    p /= p.sum()
    for s in range(steps):
        for layer in range(L_):
            ids = rng.choice(E, size=16, p=p)
            groups.append((layer * E + ids).tolist())
            plans.append(c.plan(layer, ids))
    if policy == "lru":
        h, m, v = oracle.lru(cap, groups)
    else:
        h, m, v = oracle.lfu_decay(cap, period, groups)
    assert [pl.n_hits for pl in plans] == list(h)
    assert [pl.n_misses for pl in plans] == list(m)
    st = c.stats()
    assert st["hits"] == h.sum() and st["misses"] == m.sum() and st["evictions"] == sum(len(a) for a in v)
    assert st["bytes_fetched"] == m.sum() * (1 << 20)


def test_cache_planner_hand_worked_decay_order():
    """The planner on the hand-worked sequence that fixes when counts are halved (the halving at a
    decay group comes before that group's own increments; see the oracle pins)."""
    from test_oracle_pins import LFU_HAND_GROUPS, LFU_HAND_HITS

    c = _planner(2, 1, 4, "lfu_decay", 2)
    hits, victims = [], []
    prev = {}
    for grp in LFU_HAND_GROUPS:
        pl = c.plan(0, np.array(grp))
        hits.append(pl.n_hits)
        now = {e: pl.slot_of_expert[e] for e in range(4) if pl.slot_of_expert[e] >= 0}
        victims.append(sorted(set(prev) - set(now)))
        prev = now
    assert hits == LFU_HAND_HITS
    assert victims == [[], [], [0], [1], [2], [0], []]


def test_cache_rejects_unknown_policy():
    d = _lib.MoeCacheDesc()
    d.pkg_bytes, d.L, d.E, d.capacity, d.policy = 1024, 1, 8, 4, 7
    h = ctypes.c_void_p()
    assert L.moe_cache_create(ctypes.byref(d), ctypes.byref(h)) == INVALID


def test_cache_plan_slot_table_is_injective_and_consistent():
    L_, E, cap = 2, 32, 20
    c = _planner(cap, L_, E)
    rng = np.random.default_rng(3)
    owner = {}
    for s in range(200):
        layer = s % L_
        ids = rng.integers(0, E, size=6)
        pl = c.plan(layer, ids)
        slots = [pl.slot_of_expert[e] for e in range(E)]
        for e in set(ids.tolist()):
            assert slots[e] >= 0  # every requested expert is resident after planning
        for i in range(pl.n_misses):
            owner[pl.miss_slots[i]] = (layer, pl.miss_ids[i])
        for e, sl in enumerate(slots):
            if sl >= 0:
                assert owner[sl] == (layer, e)
        used = [sl for sl in slots if sl >= 0]
        assert len(used) == len(set(used)) and all(0 <= sl < cap for sl in used)


def test_cache_plan_errors():
    c = _planner(4, 2, 16)
    with pytest.raises(moe.MoeError) as e:
        c.plan(0, np.arange(5))
    assert e.value.code == CAPACITY
    assert c.stats()["lookups"] == 0  # state unchanged
    with pytest.raises(moe.MoeError):
        c.plan(2, np.arange(2))
    with pytest.raises(moe.MoeError):
        c.plan(0, np.array([16]))
    pl = c.plan(1, np.array([3, 3, 3]))
    assert pl.n_ids == 1 and pl.n_misses == 1


def test_cache_create_rejects_unpinned_bank():
    bank = np.zeros(1 << 16, np.uint8)
    d = _lib.MoeCacheDesc()
    d.host_bank = bank.ctypes.data
    d.pkg_bytes, d.L, d.E = 1024, 1, 8
    d.device_pool = 256  # any non-null value: never dereferenced when the bank check fails
    d.slot_stride, d.capacity = 1024, 4
    h = ctypes.c_void_p()
    assert L.moe_cache_create(ctypes.byref(d), ctypes.byref(h)) == -5


def test_pack_int4_scale_domain():
    """INT4 scales must be normal binary16 values whose products with every code stay finite:
    |s| in [2^-14, 65504 / 8] (or zero); the largest bf16 below the bound and 2^-14 itself pack."""
    H = I = 32
    codes = np.zeros((I, H // 2), np.uint8)
    ok = np.full((I, 1), 0x3F80, np.uint16)  # 1.0

    def pack_with(bits):
        s = ok.copy()
        s[5, 0] = bits
        return moe.moe_pack_expert(H, I, "int4g32", {"w": [codes, codes, codes], "s": [ok, s, ok]})

    for bits in (0x45FF, 0xC5FF, 0x3880, 0x0000, 0x8000):  # 8160, -8160, 2^-14, +0, -0
        pack_with(bits)
    for bits in (0x4600, 0x4700, 0x3800, 0x0001, 0x7FC0, 0x7F80):  # 8192, 32768, 2^-15, subnormal, NaN, inf
        with pytest.raises(moe.MoeError) as e:
            pack_with(bits)
        assert e.value.code == UNSUPPORTED


def _run_planner(c, groups, kinds, L_, E):
    """Feed (layer-major keys) groups of the given kinds to the planner; per group (hits, misses, victims)."""
    out, prev = [], set()
    for keys, kind in zip(groups, kinds):
        layer = keys[0] // E
        ids = np.array([k - layer * E for k in keys], dtype=np.int32)
        fn = {"demand": c.plan, "prefetch": c.prefetch, "pin": c.pin}[kind]
        pl = fn(layer, ids)
        now = set()
        for l in range(L_):
            # every layer's table: the resident set after this call
            p2 = c.prefetch(l, np.zeros(0, np.int32))
            now |= {l * E + e for e in range(E) if p2.slot_of_expert[e] >= 0}
        out.append((pl.n_hits, pl.n_misses, sorted(prev - now)))
        prev = now
    return out


@pytest.mark.parametrize("policy,period", [("lru", 0), ("lfu_decay", 6)])
def test_planner_prefetch_and_pin_match_oracle(policy, period):
    """The planner's demand lookups, prefetches and pins against the oracle's simulator: hits,
    misses and victims of every group, and the prefetch statistics."""
    L_, E, cap = 2, 24, 10
    rng = np.random.default_rng(13)
    groups, kinds, n_pins = [], [], 0
    for g in range(300):
        layer = g % L_
        r = rng.random()
        if r < 0.03 and n_pins < 3:
            n_pins += 1
            kinds.append("pin")
            groups.append([layer * E + int(rng.integers(0, E))])
        elif r < 0.4:
            kinds.append("prefetch")
            groups.append((layer * E + rng.integers(0, E, size=3)).tolist())
        else:
            kinds.append("demand")
            groups.append((layer * E + rng.integers(0, E, size=4)).tolist())
    c = _planner(cap, L_, E, policy, period)
    got = _run_planner(c, groups, kinds, L_, E)
    h, m, v, ph = oracle.cache_sim(cap, policy, period, groups, kinds)
    assert [g[0] for g in got] == list(h)
    assert [g[1] for g in got] == list(m)
    assert [g[2] for g in got] == [sorted(a.tolist()) for a in v]
    st = c.stats()
    dem = [i for i, k in enumerate(kinds) if k == "demand"]
    assert st["hits"] == sum(h[i] for i in dem) and st["misses"] == sum(m[i] for i in dem)
    assert st["prefetch_fetches"] == sum(m[i] for i, k in enumerate(kinds) if k == "prefetch")
    assert st["prefetch_hits"] == ph
    assert st["bytes_fetched"] == m.sum() * (1 << 20)


def test_planner_hand_worked_prefetch_and_pin():
    from test_oracle_pins import (CACHE_PIN_GROUPS, CACHE_PIN_HITS, CACHE_PIN_KINDS, CACHE_PIN_VICTIMS,
                                  CACHE_PREFETCH_GROUPS, CACHE_PREFETCH_HITS, CACHE_PREFETCH_KINDS,
                                  CACHE_PREFETCH_MISSES, CACHE_PREFETCH_VICTIMS)

    got = _run_planner(_planner(3, 1, 8), CACHE_PREFETCH_GROUPS, CACHE_PREFETCH_KINDS, 1, 8)
    assert [g[0] for g in got] == CACHE_PREFETCH_HITS and [g[1] for g in got] == CACHE_PREFETCH_MISSES
    assert [g[2] for g in got] == CACHE_PREFETCH_VICTIMS
    got = _run_planner(_planner(3, 1, 8), CACHE_PIN_GROUPS, CACHE_PIN_KINDS, 1, 8)
    assert [g[0] for g in got] == CACHE_PIN_HITS and [g[2] for g in got] == CACHE_PIN_VICTIMS
    c = _planner(3, 1, 9)
    c.pin(0, np.array([7, 8]))
    with pytest.raises(moe.MoeError) as e:
        c.plan(0, np.array([0, 1]))
    assert e.value.code == CAPACITY


class FakeCopyEngine:
    """Host memcpy in place of the HIP copy engine; copy number `fail_at` (0-based) fails."""

    def __init__(self, fail_at=None):
        self.n, self.fail_at, self.log = 0, fail_at, []

    def __call__(self, dst, src, nbytes, stream):
        i = self.n
        self.n += 1
        if self.fail_at is not None and i == self.fail_at:
            return 1
        ctypes.memmove(dst, src, nbytes)
        self.log.append((dst, src, nbytes))
        return 0


def test_fetch_failure_rolls_back_and_refetches():
    """A copy that fails in the middle of a fetch: the experts whose copies did not run stop being
    resident, the next lookup misses them and fetches them again; what was copied stays valid."""
    L_, E, pkg, cap = 1, 8, 512, 4
    bank = np.random.default_rng(1).integers(0, 256, size=(E, pkg), dtype=np.uint8)
    pool = np.zeros((cap, pkg), np.uint8)
    table = np.full(E, -7, np.int32)
    eng = FakeCopyEngine(fail_at=1)
    c = ExpertCache(None, pkg, L_, E, None, pkg, cap, copy=eng, bank_ptr=bank.ctypes.data,
                    pool_ptr=pool.ctypes.data)
    p = c.plan(0, np.array([2, 5, 6]))
    assert p.n_misses == 3
    with pytest.raises(moe.MoeError) as e:
        c.fetch(p, table.ctypes.data, None)
    assert e.value.code == -3 and "not resident" in str(e.value)
    assert (table == -7).all()  # the slot table was not copied
    st = c.stats()
    assert st["bytes_fetched"] == pkg  # only the first package was copied
    eng.fail_at = None
    p = c.plan(0, np.array([2, 5, 6]))
    assert (p.n_hits, p.n_misses) == (1, 2) and sorted(p.miss_ids[i] for i in range(2)) == [5, 6]
    c.fetch(p, table.ctypes.data, None)
    for e_ in (2, 5, 6):
        assert table[e_] >= 0 and np.array_equal(pool[table[e_]], bank[e_])
    assert len(set(table[[2, 5, 6]].tolist())) == 3


# ---- lossless package compression: the library's host encoder against the oracle's

def _bf16(a):
    return (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("kind", ["gaussian", "bits", "specials", "escapes", "package"])
def test_compress_package_equals_oracle_blob(kind):
    rng = np.random.default_rng(3)
    n = 512 * 40
    if kind == "gaussian":
        v = _bf16(rng.normal(0, 0.02, n))
    elif kind == "bits":
        v = rng.integers(0, 1 << 16, n, dtype=np.uint16)
    elif kind == "specials":
        v = rng.choice(np.array([0, 0x8000, 0x7F80, 0xFF80, 0x7FC1, 0x0001, 0x8080, 0x3F80], np.uint16), n)
    elif kind == "escapes":  # chunks with 0..300 escapes around the raw-fallback boundary
        v = np.full(n, 0x5F00, np.uint16)
        for c in range(40):
            v[c * 512] = 0x6400
            v[c * 512 + 1:c * 512 + 1 + 8 * c] = 0x0080
    else:  # a real bf16 package of a small expert
        wl = W.Workload(name="cz", H=256, E=1, k=1, I=512, wfmt="bf16", xdt="bf16", Ts=(1,), seed=4)
        v = moe.moe_pack_expert(wl.H, wl.I, "bf16", W.expert_weights(wl, 0, 0)).view(np.uint16)
    raw = v.view(np.uint8)
    got = moe.moe_compress_package(raw)
    want = oracle.xw4_encode(raw)
    assert got.size == want.size and np.array_equal(got, want)
    assert np.array_equal(oracle.xw4_decode(got, raw.size), raw)
    assert moe.moe_compress_bound(raw.size) >= got.size


def test_compress_validation():
    assert moe.moe_compress_bound(1000) == 0
    assert moe.moe_compress_bound(0) == 256
    assert moe.moe_compress_bound(1 << 20) == 256 * ((64 + 4 * 1025 + 1024 + 255) // 256) + (1 << 20)
    with pytest.raises(moe.MoeError):
        moe.moe_compress_package(np.zeros(1000, np.uint8))
    with pytest.raises(moe.MoeError):
        moe.moe_compress_package(np.zeros(2048, np.uint8), out=np.zeros(100, np.uint8))
    assert moe.moe_compress_package(np.zeros(0, np.uint8)).size == 256
    # device decoder: argument checks before any pointer is touched
    assert L.moe_decompress_packages(None, 256, None, 1024, None, 1, 1000, None) == INVALID
    assert L.moe_decompress_packages(None, 100, None, 1024, None, 1, 1024, None) == INVALID
    assert L.moe_decompress_packages(None, 256, None, 512, None, 1, 1024, None) == INVALID
    assert L.moe_decompress_packages(None, 256, None, 1024, None, -1, 1024, None) == INVALID
    assert L.moe_decompress_packages(None, 256, None, 1024, None, 1, 1024, None) == INVALID  # null pointers
    assert L.moe_decompress_packages(None, 256, None, 1024, None, 0, 1024, None) == OK


# ---- order-0 rANS code: the library's host encoder against the oracle's

@pytest.mark.parametrize("kind", ["skewed", "uniform", "single", "empty_first", "empty_second", "int4", "mxfp4"])
def test_compress_rans_equals_oracle_blob(kind):
    rng = np.random.default_rng(5)
    n, q = 3 * 32768 + 999, 40000
    if kind == "skewed":
        raw = (rng.normal(0, 6, n).astype(np.int64) & 255).astype(np.uint8)
    elif kind == "uniform":
        raw = rng.integers(0, 256, n, dtype=np.uint8)
    elif kind == "single":
        raw = np.full(n, 7, np.uint8)
    elif kind in ("empty_first", "empty_second"):
        raw = (rng.normal(0, 20, n).astype(np.int64) & 255).astype(np.uint8)
        q = 0 if kind == "empty_first" else n
    else:  # a 4-bit package of a small expert, cut after its codes
        fmt = "int4g32" if kind == "int4" else "mxfp4"
        wl = W.Workload(name="cr", H=256, E=1, k=1, I=512, wfmt=fmt, xdt="bf16", Ts=(1,), seed=4)
        raw = moe.moe_pack_expert(wl.H, wl.I, fmt, W.expert_weights(wl, 0, 0))
        n, q = raw.size, moe.api.package_split(wl.H, wl.I, fmt)
        assert q == 3 * wl.H * wl.I // 2
    got = moe.moe_compress_rans(raw, q)
    want = oracle.rns_encode(raw, q)
    assert got.size == want.size and np.array_equal(got, want)
    assert np.array_equal(oracle.rns_decode(got, n), raw)
    assert moe.moe_compress_rans_bound(n) >= got.size


def test_compress_rans_validation():
    raw = np.zeros(100, np.uint8)
    with pytest.raises(moe.MoeError):
        moe.moe_compress_rans(raw, 101)  # split past the end
    with pytest.raises(moe.MoeError):
        moe.moe_compress_rans(raw, 10, out=np.zeros(1000, np.uint8))  # below the bound
    assert moe.moe_compress_rans(np.zeros(0, np.uint8), 0).size == 64 + 2 * 133648
    # device decoder: argument checks before any pointer is touched
    assert L.moe_decompress_rans(None, 100, None, 1024, None, 1, 1024, None) == INVALID
    assert L.moe_decompress_rans(None, 256, None, 512, None, 1, 1024, None) == INVALID
    assert L.moe_decompress_rans(None, 256, None, 1024, None, -1, 1024, None) == INVALID
    assert L.moe_decompress_rans(None, 256, None, 1024, None, 65536, 1024, None) == INVALID
    assert L.moe_decompress_rans(None, 256, None, 1024, None, 1, 1024, None) == INVALID  # null pointers
    assert L.moe_decompress_rans(None, 256, None, 1024, None, 0, 1024, None) == OK


def test_cache_set_rans_validation():
    """Argument checks of the rANS bank mode, all taken before any stream is created."""
    L_, E, pkg, cap = 1, 8, 512, 4
    bank = np.zeros((E, pkg), np.uint8)
    pool = np.zeros((cap, 1024), np.uint8)
    c = ExpertCache(None, pkg, L_, E, None, 1024, cap, copy=FakeCopyEngine(), bank_ptr=bank.ctypes.data,
                    pool_ptr=pool.ctypes.data)
    st = ctypes.c_void_p(0x1000)
    assert L.moe_cache_set_rans(c.h, None, 512, 4, 1024) == INVALID        # no staging
    assert L.moe_cache_set_rans(c.h, st, 256, 4, 1024) == INVALID          # staging slot below pkg_bytes
    assert L.moe_cache_set_rans(c.h, st, 600, 4, 1024) == INVALID          # not a multiple of 256
    assert L.moe_cache_set_rans(c.h, st, 512, 0, 1024) == INVALID          # no staging slots
    assert L.moe_cache_set_rans(c.h, st, 512, 65, 1024) == INVALID
    assert L.moe_cache_set_rans(c.h, st, 512, 4, 1025) == INVALID          # package larger than a pool slot
    assert L.moe_cache_set_rans(c.h, st, 512, 4, 0) == INVALID
    assert L.moe_cache_set_rans(None, st, 512, 4, 1024) == INVALID
    planning = ExpertCache(None, 1 << 20, L_, E, None, 0, cap)
    assert L.moe_cache_set_rans(planning.h, st, 1 << 20, 4, 1024) == INVALID  # no bank
