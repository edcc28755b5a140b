"""Pins for the CPU oracle, each independent of the oracle's own code.

Decoders are checked against literal code tables (OCP MX v1.0 for E2M1/E8M0,
two's complement for INT4) and numpy's own float views; the router against a
numpy fp64 matmul; top-k against a full lexicographic sort; the permutation
against numpy's stable argsort; the expert FFN against a dense torch fp64
SwiGLU; the layer against invariants that the definition fixes (identical
experts give the dense FFN whatever the routing, token order and expert labels
do not matter, the shared expert adds with weight 1) and a brute-force numpy
evaluation of the tiny layer; the caches against an OrderedDict LRU and a
brute-force optimum.
"""
import itertools
import math
from collections import OrderedDict

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import workloads as W

# OCP Microscaling Formats v1.0, FP4 E2M1: codes 0..15 -> value
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
INT4_TABLE = [0, 1, 2, 3, 4, 5, 6, 7, -8, -7, -6, -5, -4, -3, -2, -1]


def bf16_to_f64(h):
    return (np.asarray(h, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16_bits_trunc(v):
    return (np.asarray(v, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


# ------------------------------------------------------------------ decoders

def test_mxfp4_decoder_exhaustive():
    # one row, K = 32 * 256: block b has E8M0 scale b (0..254; 255 is NaN), elements cycle all 16 codes
    K = 32 * 255
    codes = np.zeros((1, K // 2), dtype=np.uint8)
    for i in range(K // 2):
        lo, hi = (2 * i) % 16, (2 * i + 1) % 16
        codes[0, i] = lo | (hi << 4)
    scales = np.arange(255, dtype=np.uint8).reshape(1, 255)
    got = oracle.decode("mxfp4", codes, scales, 1, K)[0]
    for k in range(K):
        want = E2M1_TABLE[k % 16] * math.ldexp(1.0, (k // 32) - 127)
        assert got[k] == want and math.copysign(1, got[k]) == math.copysign(1, want), k


def test_mxfp4_nan_scale():
    codes = np.full((1, 16), 0x21, dtype=np.uint8)
    got = oracle.decode("mxfp4", codes, np.array([[255]], dtype=np.uint8), 1, 32)
    assert np.isnan(got).all()


def test_int4_decoder_exhaustive():
    scale_vals = [1.0, 0.0078125, 3.0, -0.5, 2.0 ** -20, 1.5 * 2.0 ** 10, 0.0, 0.021484375]
    sb = f64_to_bf16_bits_trunc(scale_vals)
    assert np.all(bf16_to_f64(sb) == np.array(scale_vals))
    K = 32 * len(scale_vals)
    codes = np.zeros((1, K // 2), dtype=np.uint8)
    for i in range(K // 2):
        codes[0, i] = ((2 * i) % 16) | (((2 * i + 1) % 16) << 4)
    got = oracle.decode("int4g32", codes, sb.reshape(1, -1), 1, K)[0]
    for k in range(K):
        assert got[k] == INT4_TABLE[k % 16] * scale_vals[k // 32], k


def test_plain_decoders_match_numpy_views():
    rng = np.random.default_rng(0)
    f = rng.standard_normal((7, 64)).astype(np.float32)
    assert np.array_equal(oracle.decode("f32", f, None, 7, 64), f.astype(np.float64))
    h = rng.integers(0, 65536, size=(5, 32), dtype=np.uint16)
    h[(h & 0x7F80) == 0x7F80] = 0x3F80  # no inf/nan patterns
    assert np.array_equal(oracle.decode("bf16", h, None, 5, 32), bf16_to_f64(h))
    assert np.array_equal(oracle.decode_act("bf16", h), bf16_to_f64(h))


def test_nibble_order_low_first():
    codes = np.array([[0x71] + [0] * 15], dtype=np.uint8)  # element 0 = code 1 (0.5), element 1 = code 7 (6)
    got = oracle.decode("mxfp4", codes, np.array([[127]], dtype=np.uint8), 1, 32)[0]
    assert got[0] == 0.5 and got[1] == 6.0 and not got[2:].any()


# -------------------------------------------------------------------- router

def test_router_logits_vs_numpy():
    rng = np.random.default_rng(1)
    T, H, E = 9, 96, 11
    x = rng.standard_normal((T, H)).astype(np.float32)
    wg = (0.1 * rng.standard_normal((E, H))).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    got = oracle.router_logits("f32", x, wg, b)
    want = x.astype(np.float64) @ wg.astype(np.float64).T + b.astype(np.float64)
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)
    xb = f64_to_bf16_bits_trunc(rng.standard_normal((T, H)))
    wb = f64_to_bf16_bits_trunc(0.1 * rng.standard_normal((E, H)))
    got = oracle.router_logits("bf16", xb, wb, None)
    np.testing.assert_allclose(got, bf16_to_f64(xb) @ bf16_to_f64(wb).T, rtol=1e-13, atol=1e-13)


def test_topk_brute_force_and_gates():
    rng = np.random.default_rng(2)
    T, E = 50, 13
    lg = rng.standard_normal((T, E))
    lg[3, 4] = lg[3, 9] = 5.0  # exact tie at the top: lower id first
    lg[7, :] = 0.25  # all tied
    for k in (1, 3, E):
        ids, w = oracle.topk_gates(lg, k)
        for t in range(T):
            order = sorted(range(E), key=lambda e: (-lg[t, e], e))[:k]
            assert list(ids[t]) == order
            full = np.exp(lg[t] - lg[t].max())
            full /= full.sum()  # softmax over all E
            ren = full[order] / full[order].sum()  # renormalised over the chosen k
            np.testing.assert_allclose(w[t], ren, rtol=1e-14, atol=1e-15)
            assert abs(w[t].sum() - 1.0) < 1e-14
            assert np.all(np.diff(w[t]) <= 1e-15)
    ids, _ = oracle.topk_gates(lg, 2)
    assert list(ids[3]) == [4, 9]
    assert list(ids[7]) == [0, 1]


def test_topk_k1_weight_is_one():
    lg = np.random.default_rng(3).standard_normal((20, 8))
    ids, w = oracle.topk_gates(lg, 1)
    assert np.array_equal(ids[:, 0], lg.argmax(axis=1)) and np.all(w == 1.0)


# --------------------------------------------------------------- permutation

@pytest.mark.parametrize("T,k,E", [(0, 2, 8), (1, 1, 1), (16, 2, 8), (333, 8, 384), (64, 4, 128), (5, 8, 8)])
def test_permute_vs_stable_argsort(T, k, E):
    rng = np.random.default_rng(T * 31 + k)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32) if T else np.zeros((0, k), np.int32)
    counts, offsets, perm, inv = oracle.permute(ids, E)
    flat = ids.ravel()
    assert np.array_equal(perm, np.argsort(flat, kind="stable"))
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts) and offsets[-1] == T * k
    assert np.array_equal(inv[perm], np.arange(T * k))
    # each token appears exactly k times; inside an expert the tokens ascend
    assert np.array_equal(np.bincount(perm // k, minlength=T) if T else np.zeros(0), np.full(T, k))
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)


def test_permute_all_on_one_expert():
    ids = np.full((10, 1), 3, dtype=np.int32)
    counts, offsets, perm, inv = oracle.permute(ids, 5)
    assert list(counts) == [0, 0, 0, 10, 0] and list(offsets) == [0, 0, 0, 0, 10, 10]
    assert np.array_equal(perm, np.arange(10))


# ------------------------------------------------------------------- expert FFN

def dense_swiglu_torch(x, g, u, d):
    x, g, u, d = (torch.from_numpy(np.asarray(a, dtype=np.float64)) for a in (x, g, u, d))
    return (torch.nn.functional.silu(x @ g.T) * (x @ u.T) @ d.T).numpy()


@pytest.mark.parametrize("fmt", ["f32", "bf16", "mxfp4", "int4g32"])
def test_ffn_equals_dense_swiglu(fmt):
    wl = W.WORKLOADS["tiny"].with_(wfmt=fmt, H=64, I=96, name="ffn-pin-" + fmt)
    ex = W.expert_weights(wl, 0, 0)
    dec = [oracle.decode(fmt, ex["w"][m], ex["s"][m], *shape)
           for m, shape in enumerate([(wl.I, wl.H), (wl.I, wl.H), (wl.H, wl.I)])]
    x = np.random.default_rng(4).standard_normal((5, wl.H))
    got = oracle.ffn(ex, wl.H, wl.I, x)
    np.testing.assert_allclose(got, dense_swiglu_torch(x, *dec), rtol=1e-12, atol=1e-14)


# -------------------------------------------------------------------- layer

def _tiny(fmt="f32", **kw):
    return W.WORKLOADS["tiny"].with_(wfmt=fmt, name="pin-" + fmt, **kw)


def _layer_inputs(wl, T):
    x = W.activations(wl, T)
    wg = W.router_weights(wl)
    bias = W.router_bias(wl)
    experts = [W.expert_weights(wl, 0, e) for e in range(wl.E)]
    return x, wg, bias, experts


def test_layer_brute_force_numpy():
    wl = _tiny()
    T = 16
    x, wg, bias, experts = _layer_inputs(wl, T)
    out, ids, w = oracle.moe_layer("f32", x, wg, bias, wl.k, wl.I, experts)
    xd = x.astype(np.float64)
    logits = xd @ wg.astype(np.float64).T
    for t in range(T):
        order = np.lexsort((np.arange(wl.E), -logits[t]))[:wl.k]
        assert list(ids[t]) == list(order)
        p = np.exp(logits[t, order] - logits[t, order].max())
        p /= p.sum()
        acc = np.zeros(wl.H)
        for j, e in enumerate(order):
            g, u, d = (experts[e]["w"][m].astype(np.float64) for m in range(3))
            z = g @ xd[t]
            acc += p[j] * (d @ (z / (1 + np.exp(-z)) * (u @ xd[t])))
        np.testing.assert_allclose(out[t], acc, rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("fmt", ["f32", "bf16", "mxfp4", "int4g32"])
def test_layer_identical_experts_is_dense(fmt):
    wl = _tiny(fmt, zipf_s=1.1)
    x, wg, bias, experts = _layer_inputs(wl, 12)
    same = [experts[0]] * wl.E
    out, ids, _ = oracle.moe_layer(wl.xdt, x, wg, bias, wl.k, wl.I, same)
    assert len(set(ids.ravel().tolist())) > 1
    dense = oracle.ffn(experts[0], wl.H, wl.I, oracle.decode_act(wl.xdt, x))
    np.testing.assert_allclose(out, dense, rtol=1e-12, atol=1e-14)


def test_layer_token_permutation_equivariance():
    wl = _tiny()
    x, wg, bias, experts = _layer_inputs(wl, 16)
    out, ids, w = oracle.moe_layer("f32", x, wg, bias, wl.k, wl.I, experts)
    p = np.random.default_rng(5).permutation(16)
    out2, ids2, w2 = oracle.moe_layer("f32", np.ascontiguousarray(x[p]), wg, bias, wl.k, wl.I, experts)
    assert np.array_equal(out2, out[p]) and np.array_equal(ids2, ids[p])


def test_layer_expert_relabelling_invariance():
    wl = _tiny("bf16", zipf_s=1.1)
    x, wg, bias, experts = _layer_inputs(wl, 16)
    out, ids, _ = oracle.moe_layer("f32", x, wg, bias, wl.k, wl.I, experts)
    p = np.random.default_rng(6).permutation(wl.E)
    out2, ids2, _ = oracle.moe_layer("f32", x, np.ascontiguousarray(wg[p]), np.ascontiguousarray(bias[p]), wl.k,
                                     wl.I, [experts[q] for q in p])
    np.testing.assert_allclose(out2, out, rtol=1e-13, atol=1e-15)
    assert np.array_equal(p[ids2], ids)


def test_layer_sampling_and_shared_expert():
    wl = _tiny("bf16", shared=True, xdt="bf16")
    x, wg, bias, experts = _layer_inputs(wl, 16)
    sh = W.shared_weights(wl)
    full, ids, w = oracle.moe_layer("bf16", x, wg, bias, wl.k, wl.I, experts)
    s = np.array([11, 2, 7])
    part, ids_s, w_s = oracle.moe_layer("bf16", x, wg, bias, wl.k, wl.I, experts, sample=s)
    np.testing.assert_array_equal(part, full[s])
    assert np.array_equal(ids_s, ids[s]) and np.array_equal(w_s, w[s])
    with_sh, _, _ = oracle.moe_layer("bf16", x, wg, bias, wl.k, wl.I, experts, shared=sh, I_shared=wl.I)
    dec = [oracle.decode("bf16", sh["w"][m], None, *shape)
           for m, shape in enumerate([(wl.I, wl.H), (wl.I, wl.H), (wl.H, wl.I)])]
    np.testing.assert_allclose(with_sh - full, dense_swiglu_torch(oracle.decode_act("bf16", x), *dec),
                               rtol=1e-9, atol=1e-12)


def test_rank_gap_inputs():
    wl = _tiny()
    x, attempts = oracle.rank_gap_inputs(wl, 16)
    lg = oracle.router_logits("f32", x, W.router_weights(wl), None)
    assert oracle.min_gap(lg, wl.k).min() >= 1e-3
    x0 = W.activations(wl, 16)
    same = attempts == 0
    assert np.array_equal(x[same], x0[same])


# --------------------------------------------------------------------- caches

def lru_ordered_dict(capacity, groups):
    od = OrderedDict()
    hits, misses, victims = [], [], []
    for grp in groups:
        cur = sorted(set(int(v) for v in grp))
        h = m = 0
        vic = []
        for key in cur:
            if key in od:
                h += 1
                od.move_to_end(key)
            else:
                m += 1
                if len(od) == capacity:
                    victim = next(c for c in od if c not in cur)
                    del od[victim]
                    vic.append(victim)
                od[key] = True
        hits.append(h)
        misses.append(m)
        victims.append(vic)
    return hits, misses, victims


def _zipf_groups(n_groups, per_group, space, seed):
    rng = np.random.default_rng(seed)
    p = 1.0 / np.arange(1, space + 1) ** 1.2
    p /= p.sum()
    return [rng.choice(space, size=per_group, p=p) for _ in range(n_groups)]


@pytest.mark.parametrize("cap,per,space,seed", [(4, 2, 12, 0), (16, 8, 64, 1), (32, 16, 256, 2), (8, 8, 9, 3)])
def test_lru_vs_ordered_dict(cap, per, space, seed):
    groups = _zipf_groups(300, per, space, seed)
    h, m, v = oracle.lru(cap, groups)
    h2, m2, v2 = lru_ordered_dict(cap, groups)
    assert list(h) == h2 and list(m) == m2
    assert [list(a) for a in v] == v2
    for g, grp in enumerate(groups):
        assert h[g] + m[g] == len(set(grp.tolist()))


def test_lru_capacity_error():
    with pytest.raises(ValueError):
        oracle.lru(2, [[1, 2, 3]])


def _opt_hits_brute(capacity, groups):
    """Largest hit count over every eviction choice (tiny inputs only)."""
    best = 0

    def rec(g, resident, hits):
        nonlocal best
        if g == len(groups):
            best = max(best, hits)
            return
        cur = sorted(set(groups[g]))
        h = sum(1 for c in cur if c in resident)
        miss = [c for c in cur if c not in resident]
        others = sorted(resident - set(cur))
        need = max(0, len(resident) + len(miss) - capacity)
        for ev in itertools.combinations(others, need):
            rec(g + 1, (resident - set(ev)) | set(miss), hits + h)

    rec(0, frozenset(), 0)
    return best


@pytest.mark.parametrize("seed", range(6))
def test_belady_is_optimal_on_tiny_inputs(seed):
    groups = [list(g) for g in _zipf_groups(9, 2, 6, 100 + seed)]
    hb, mb = oracle.belady(3, groups)
    assert hb.sum() == _opt_hits_brute(3, groups)
    hl, ml, _ = oracle.lru(3, groups)
    assert hb.sum() >= hl.sum() and (hb + mb == hl + ml).all()


@pytest.mark.parametrize("cap,space,seed", [(4, 12, 0), (16, 64, 1), (33, 256, 2)])
def test_lfu_decay_with_period_one_is_lru_on_single_key_groups(cap, space, seed):
    """Halving every group makes the most recent use dominate every count (a use one group ago
    outweighs all older uses together), so with one key per group (no ties in last use) the
    eviction order is exactly least-recently-used."""
    groups = [[int(k)] for k in np.concatenate(_zipf_groups(600, 1, space, seed))]
    h, m, v = oracle.lfu_decay(cap, 1, groups)
    h2, m2, v2 = lru_ordered_dict(cap, groups)
    assert list(h) == h2 and list(m) == m2
    assert [list(a) for a in v] == v2


def test_lfu_decay_keeps_a_hot_set_that_lru_loses():
    """Without decay, keys used again and again outrank one-off keys: four hot keys come back
    every third group, two bursts of six new keys come between.  With 12 slots LRU evicts the
    hot keys every time (the 12 keys of the two bursts are all more recent); frequency keeps
    them resident once their counts exceed a one-off key's."""
    hot = list(range(4))
    groups, nxt = [], 100
    for g in range(90):
        if g % 3 == 0:
            groups.append(list(hot))
        else:
            groups.append(list(range(nxt, nxt + 6)))
            nxt += 6
    hl, ml, _ = oracle.lfu_decay(12, 0, groups)
    hr, mr, _ = oracle.lru(12, groups)
    assert all(hl[g] == 4 for g in range(9, 90, 3))
    assert all(hr[g] == 0 for g in range(3, 90, 3))
    assert (hl + ml == hr + mr).all()


# A hand-worked sequence that fixes when the counts are halved: at the start of a decay group,
# before that group's keys gain their 1024.  Capacity 2, period 2, keys a=0 b=1 c=2 d=3, one key
# per group: [a] [b] [c] [a] [d] [b] [d].  Counts (before each group's lookups) and the victim
# chosen by the smallest (count, last use, key) among resident keys not in the group:
#   g0 a=1024                                   miss
#   g1 b=1024                                   miss
#   g2 halve: a=512 b=512;   c=1024             miss, a (512, last 0) < b (512, last 1): evict a
#   g3 a=512+1024=1536                          miss, b (512) < c (1024): evict b
#   g4 halve: a=768 b=256 c=512; d=1024         miss, c (512) < a (768): evict c
#   g5 b=256+1024=1280                          miss, a (768) < d (1024): evict a
#   g6 halve: a=384 b=640 c=256 d=512; d=1536   d resident: hit
# Halving after the group's own increment would give d (1024 + 0) / 2 = 512 at g4 and evict d at g5
# (then miss at g6); no decay at all would also evict d at g5 (a=2048 > d=1024).
LFU_HAND_GROUPS = [[0], [1], [2], [0], [3], [1], [3]]
LFU_HAND_HITS = [0, 0, 0, 0, 0, 0, 1]
LFU_HAND_VICTIMS = [[], [], [0], [1], [2], [0], []]


def test_lfu_decay_hand_worked_order_of_halving():
    h, m, v = oracle.lfu_decay(2, 2, LFU_HAND_GROUPS)
    assert list(h) == LFU_HAND_HITS
    assert list(m) == [1 - x for x in LFU_HAND_HITS]
    assert [list(a) for a in v] == LFU_HAND_VICTIMS


@pytest.mark.parametrize("policy,period", [("lru", 0), ("lfu_decay", 0), ("lfu_decay", 5)])
def test_cache_sim_demand_only_equals_the_plain_policies(policy, period):
    """With demand groups only, the simulator with prefetch and pin kinds is the plain policy."""
    groups = [list(g) for g in _zipf_groups(300, 8, 64, 21)]
    h, m, v, ph = oracle.cache_sim(16, policy, period, groups, ["demand"] * len(groups))
    h2, m2, v2 = oracle.lru(16, groups) if policy == "lru" else oracle.lfu_decay(16, period, groups)
    assert list(h) == list(h2) and list(m) == list(m2) and [list(a) for a in v] == [list(a) for a in v2]
    assert ph == 0


# Hand-worked prefetch sequence, capacity 3, LRU (ticks count demand groups only):
#   g0 demand  [0 1]   misses 0, 1 (tick 0)
#   g1 prefetch [2 3]  2 takes the free slot (last use -1); 3 would need a victim outside {2, 3} and
#                      the latest demand group {0, 1}: none, so it is skipped
#   g2 demand  [2 4]   2 hits (a prefetch hit); 4 evicts the smallest (last, key) outside {2, 4}:
#                      0 (last 0) before 1 (last 0, larger key)          (tick 1)
#   g3 prefetch [5]    victim outside {5} and {2, 4}: 1; 5 enters with last use -1
#   g4 demand  [0]     victim among 2 (last 1), 4 (last 1), 5 (last -1): 5, the unused prefetch
CACHE_PREFETCH_GROUPS = [[0, 1], [2, 3], [2, 4], [5], [0]]
CACHE_PREFETCH_KINDS = ["demand", "prefetch", "demand", "prefetch", "demand"]
CACHE_PREFETCH_HITS = [0, 0, 1, 0, 0]
CACHE_PREFETCH_MISSES = [2, 1, 1, 1, 1]
CACHE_PREFETCH_VICTIMS = [[], [], [0], [1], [5]]

# Hand-worked pin sequence, capacity 3, LRU:
#   g0 pin     [7]     7 fetched and pinned
#   g1 demand  [0 1]   misses (tick 0)
#   g2 demand  [2]     victim among 0, 1 (7 is pinned): 0                   (tick 1)
#   g3 demand  [7 3]   7 hits; 3 evicts 1 (last 0) before 2 (last 1)        (tick 2)
#   g4 demand  [4 5]   two misses; 7 is pinned, so 2 (last 1) then 3 (last 2) go         (tick 3)
CACHE_PIN_GROUPS = [[7], [0, 1], [2], [7, 3], [4, 5]]
CACHE_PIN_KINDS = ["pin", "demand", "demand", "demand", "demand"]
CACHE_PIN_HITS = [0, 0, 0, 1, 0]
CACHE_PIN_VICTIMS = [[], [], [0], [1], [2, 3]]


def test_cache_sim_hand_worked_prefetch():
    h, m, v, ph = oracle.cache_sim(3, "lru", 0, CACHE_PREFETCH_GROUPS, CACHE_PREFETCH_KINDS)
    assert list(h) == CACHE_PREFETCH_HITS and list(m) == CACHE_PREFETCH_MISSES
    assert [list(a) for a in v] == CACHE_PREFETCH_VICTIMS
    assert ph == 1


def test_cache_sim_hand_worked_pin():
    h, m, v, ph = oracle.cache_sim(3, "lru", 0, CACHE_PIN_GROUPS, CACHE_PIN_KINDS)
    assert list(h) == CACHE_PIN_HITS
    assert [list(a) for a in v] == CACHE_PIN_VICTIMS
    # a demand group that needs more slots than the pin leaves is refused
    with pytest.raises(ValueError):
        oracle.cache_sim(3, "lru", 0, [[7, 8], [0, 1]], ["pin", "demand"])


@pytest.mark.parametrize("policy,period", [("lru", 0), ("lfu_decay", 7)])
def test_cache_sim_invariants_random(policy, period):
    """Random mixes: a pinned key is never a victim; a prefetch never evicts a key of the latest
    demand group; hits + misses of a demand group = its distinct keys; a prefetch fetches at most
    its absent keys."""
    rng = np.random.default_rng(5)
    groups, kinds, pinned = [], [], set()
    n_pins = 0
    for g in range(400):
        r = rng.random()
        if r < 0.02 and n_pins < 4:  # (at most 4 pinned keys: every demand group of 4 still fits 12 slots)
            n_pins += 1
            kinds.append("pin")
            groups.append([int(rng.integers(0, 40))])
        elif r < 0.35:
            kinds.append("prefetch")
            groups.append(rng.integers(0, 40, size=3).tolist())
        else:
            kinds.append("demand")
            groups.append(rng.integers(0, 40, size=4).tolist())
    cap = 12
    h, m, v, ph = oracle.cache_sim(cap, policy, period, groups, kinds)
    last_demand = set()
    for g, (grp, kind) in enumerate(zip(groups, kinds)):
        assert not (set(v[g].tolist()) & pinned)
        if kind == "prefetch":
            assert not (set(v[g].tolist()) & last_demand)
            assert m[g] <= len(set(grp))
        if kind == "demand":
            assert h[g] + m[g] == len(set(grp))
            last_demand = set(grp)
        if kind == "pin":
            pinned |= set(grp)
        assert not (set(v[g].tolist()) & set(grp))


def test_belady_at_least_lru_large():
    groups = _zipf_groups(400, 16, 512, 7)
    hb, _ = oracle.belady(64, groups)
    hl, _, _ = oracle.lru(64, groups)
    hf, _, _ = oracle.lfu_decay(64, 32, groups)
    assert hb.sum() >= hl.sum() and hb.sum() >= hf.sum()


# ------------------------------------------------------------- cost model (report formula)

def test_cost_model_matches_the_printed_worked_example():
    """T = C + S, S = B / W: the GLM and Kimi figures of the Galactus cost model."""
    import json
    import os

    import bench

    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "galactus_cost_model.json")))
    k = g["kimi_streaming"]
    assert abs(bench.streaming_time(k["B_bytes"], k["W_bytes_per_s"]) - k["S_s_approx"]) < 1e-9
    r = g["glm_rounded"]
    cm = bench.cost_model(r["C_s"], r["S_s"])
    assert abs(cm["T_s"] - r["T_s"]) < 1e-12 and round(cm["tokens_per_s"], 2) == r["tokens_per_s"]
    m = g["glm_traffic_minus_25pct"]
    S2 = round(r["S_s"] * 0.75, 3)  # "about 68 ms"
    assert abs(S2 - m["S_s_approx"]) < 1e-9
    cm2 = bench.cost_model(r["C_s"], S2)
    assert abs(cm2["T_s"] - m["T_s_approx"]) < 1e-9 and round(cm2["tokens_per_s"], 2) == m["tokens_per_s"]
    assert round(cm2["tokens_per_s"] / cm["tokens_per_s"] - 1, 2) == m["gain_approx"]
    mr = g["measured_reciprocals"]
    assert round(1000 / mr["kimi_tok_s"]) == mr["kimi_ms"] and round(1000 / mr["glm_tok_s"]) == mr["glm_ms"]


# ---- lossless exponent-window code of bf16 packages (the definition is in oracle.c)

def _chunk(vals):
    v = np.asarray(vals, np.uint16)
    assert v.size == 512
    return v.view(np.uint8)


def test_xw4_hand_worked_chunk():
    """One chunk, worked by hand from the definition: values -2.0 (0xC000), +0, 1.5 (0x3FC0), the
    smallest negative subnormal (0x8001), then 508 x 1.0 (0x3F80).  Largest exponent field 128, so
    the window base is 114: -2.0 -> code 15, 1.0 and 1.5 -> code 14, the two exponent-0 values are
    escapes (code 0, escape bytes 0x00 0x00).  Coded size 768 + 16; the tables take 64 + 8 + 1
    bytes, so the data starts at 256 and the blob is 1040 bytes."""
    raw = _chunk([0xC000, 0x0000, 0x3FC0, 0x8001] + [0x3F80] * 508)
    blob = oracle.xw4_encode(raw)
    assert blob.size == 1040
    hdr = blob[:64]
    assert hdr[:4].tobytes() == bytes([0x58, 0x57, 0x34, 0x31])
    assert int.from_bytes(hdr[4:8].tobytes(), "little") == 1
    assert int.from_bytes(hdr[8:16].tobytes(), "little") == 1024
    assert int.from_bytes(hdr[16:24].tobytes(), "little") == 256
    assert int.from_bytes(hdr[24:32].tobytes(), "little") == 1040
    assert not hdr[32:].any()
    assert blob[64:72].view(np.uint32).tolist() == [0, 784]
    assert blob[72] == 114
    assert not blob[73:256].any()
    d = blob[256:]
    sm = [0x80, 0x00, 0x40, 0x81] + [0x00] * 508
    codes = [0x0F, 0x0E] + [0xEE] * 254
    assert d[:512].tolist() == sm
    assert d[512:768].tolist() == codes
    assert d[768:784].tolist() == [0] * 16
    assert np.array_equal(oracle.xw4_decode(blob, 1024), raw)


@pytest.mark.parametrize("n_esc,raw_chunk", [(0, False), (1, False), (16, False), (17, False), (240, False),
                                             (241, True), (400, True)])
def test_xw4_escape_count_and_raw_fallback(n_esc, raw_chunk):
    """Largest exponent 200 (0x6400) puts the window at 186..200; exponent-1 values (0x0080) escape
    and exponent-190 values (0x5F00) do not.  A chunk is coded while 768 + 16 ceil(n_esc / 16) < 1024
    (at most 240 escapes) and stored raw from there on."""
    vals = [0x6400] + [0x0080] * n_esc + [0x5F00] * (511 - n_esc)
    raw = _chunk(vals)
    blob = oracle.xw4_encode(raw)
    size = int(blob[68:72].view(np.uint32)[0])
    if raw_chunk:
        assert size == 1024 and blob[72] == 0
        assert np.array_equal(blob[256:256 + 1024], raw)
    else:
        assert size == 768 + 16 * ((n_esc + 15) // 16)
        assert blob[72] == 186
        d = blob[256:]
        assert d[768:768 + n_esc].tolist() == [1] * n_esc  # the escaped exponent fields, in value order
        c = np.concatenate([d[512:768] & 15, d[512:768] >> 4], axis=0).reshape(2, 256).T.ravel()
        assert c[0] == 15 and (c[1:1 + n_esc] == 0).all() and (c[1 + n_esc:] == 5).all()
    assert np.array_equal(oracle.xw4_decode(blob, 1024), raw)


def test_xw4_small_exponents_window_starts_at_zero():
    """Largest exponent below 14: the window is 0..14, so zeros and subnormals are coded (code 1)."""
    raw = _chunk([0x0000, 0x8000, 0x0001, 0x0680] + [0x0000] * 508)  # +0, -0, subnormal, exponent 13
    blob = oracle.xw4_encode(raw)
    assert blob.size == 256 + 768 and blob[72] == 0
    c = blob[256 + 512:256 + 768]
    assert c[0] == 0x11 and c[1] == 0xE1 and (c[2:] == 0x11).all()
    assert np.array_equal(oracle.xw4_decode(blob, 1024), raw)


def _bf16_bits(a):
    return (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)  # truncation: any bf16 value


@pytest.mark.parametrize("kind", ["normal", "uniform_bits", "specials", "mixed"])
def test_xw4_round_trip_is_exact(kind):
    rng = np.random.default_rng(11)
    n = 512 * 24
    if kind == "normal":
        v = _bf16_bits(rng.normal(0, 0.02, n))
    elif kind == "uniform_bits":
        v = rng.integers(0, 1 << 16, n, dtype=np.uint16)
    elif kind == "specials":
        pool = np.array([0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0x7FFF, 0xFFC1, 0x0001, 0x807F, 0x0080, 0x7F7F,
                         0xFF7F, 0x3F80], np.uint16)
        v = rng.choice(pool, n)
    else:
        v = _bf16_bits(rng.normal(0, 0.02, n))
        v[rng.integers(0, n, 300)] = rng.integers(0, 1 << 16, 300, dtype=np.uint16)
        v[5 * 512:6 * 512] = 0
    raw = v.view(np.uint8)
    blob = oracle.xw4_encode(raw)
    assert np.array_equal(oracle.xw4_decode(blob, raw.size), raw)
    # chunk sizes from the definition, counted with numpy: 768 + 16 ceil(escapes / 16), or raw 1024
    e = ((v.reshape(-1, 512) >> 7) & 255).astype(np.int64)
    b = np.maximum(e.max(axis=1) - 14, 0)
    esc = ((e < b[:, None]) | (e > b[:, None] + 14)).sum(axis=1)
    coded = 768 + 16 * ((esc + 15) // 16)
    want = np.where(coded < 1024, coded, 1024)
    off = blob[64:64 + 4 * 25].view(np.uint32)
    assert np.array_equal(np.diff(off.astype(np.int64)), want)
    assert blob.size == 256 + want.sum()


def test_xw4_ratio_on_gaussian_weights():
    """N(0, 0.02) bf16 weights: 12 bits per value plus rare escapes, about 75% of the package."""
    rng = np.random.default_rng(5)
    raw = _bf16_bits(rng.normal(0, 0.02, 512 * 2048)).view(np.uint8)
    blob = oracle.xw4_encode(raw)
    assert 0.75 <= blob.size / raw.size < 0.76


def test_xw4_decode_rejects_malformed_blobs():
    raw = _chunk([0x3F80] * 512)
    blob = oracle.xw4_encode(raw)
    assert np.array_equal(oracle.xw4_decode(blob, 1024), raw)
    for mutate in (lambda b: b.__setitem__(0, 0), lambda b: b.__setitem__(4, 2),
                   lambda b: b.__setitem__(68, 0x10)):
        bad = blob.copy()
        mutate(bad)
        with pytest.raises(ValueError):
            oracle.xw4_decode(bad, 1024)
    with pytest.raises(ValueError):
        oracle.xw4_decode(blob, 2048)
    with pytest.raises(ValueError):
        oracle.xw4_decode(blob[:600], 1024)
    with pytest.raises(ValueError):
        oracle.xw4_encode(np.zeros(1000, np.uint8))


# ---- order-0 rANS code of packages (the definition is in oracle.c)

RNS_S = 32768
RNS_G = RNS_S // 64
RNS_REGION_HEAD = 512 + 4 * RNS_S + 4 * (RNS_G + 1)


def _rns_region(blob, off):
    f = blob[off:off + 512].view(np.uint16)
    states = blob[off + 512:off + 512 + 4 * RNS_S].view(np.uint32)
    offs = blob[off + 512 + 4 * RNS_S:off + RNS_REGION_HEAD].view(np.uint32)  # per group of 64 streams
    return f, states, offs


def test_rns_hand_worked_region():
    """Bytes [0, 0, 1] as one region, worked by hand: h = {0: 2, 1: 1}, m = 3, so f[0] = floor(8192/3)
    = 2730 and f[1] = 1365 sum to 4095 and the larger, f[0], takes the missing one: 2731; c[1] = 2731.
    Streams 0, 1, 2 hold one symbol each.  From x = 65536 no word is emitted (65536 < 2^20 f), and
    x = 4096 (x div f) + (x mod f) + c: symbol 0 -> 4096 * 23 + 2723 = 96931, symbol 1 -> 4096 * 48 +
    16 + 2731 = 199355.  Every other stream keeps 65536; no words; each region section is
    512 + 4 * 32768 + 4 * 513 = 133636 bytes padded to 133648; the second region is empty."""
    raw = np.array([0, 0, 1], np.uint8)
    blob = oracle.rns_encode(raw, 3)
    assert blob.size == 64 + 2 * 133648
    assert blob[:4].tobytes() == bytes([0x52, 0x4E, 0x53, 0x31])
    assert blob[4:8].view(np.uint32)[0] == RNS_S
    assert blob[8:16].view(np.uint64)[0] == 3 and blob[16:24].view(np.uint64)[0] == 3
    assert blob[24:32].view(np.uint64)[0] == blob.size
    f, states, offs = _rns_region(blob, 64)
    assert f[0] == 2731 and f[1] == 1365 and f[2:].sum() == 0
    assert states[:3].tolist() == [96931, 96931, 199355]
    assert (states[3:] == 65536).all() and (offs == 0).all()
    f2, states2, offs2 = _rns_region(blob, 64 + 133648)
    assert f2.sum() == 0 and (states2 == 65536).all() and (offs2 == 0).all()
    assert np.array_equal(oracle.rns_decode(blob, 3), raw)


@pytest.mark.parametrize("kind", ["single", "uniform256", "rare"])
def test_rns_model_normalisation(kind):
    """Frequencies sum to 4096 with every present byte at least 1: a single byte value takes all
    4096; 256 equally frequent values take 16 each; a value seen once in 10,000 bytes gets 1 and
    the largest value gives up the excess."""
    if kind == "single":
        raw, want = np.full(1000, 7, np.uint8), {7: 4096}
    elif kind == "uniform256":
        raw, want = np.tile(np.arange(256, dtype=np.uint8), 40), {s: 16 for s in range(256)}
    else:
        raw = np.zeros(10000, np.uint8)
        raw[:6000] = 3
        raw[6000:9999] = 9
        raw[9999] = 200
        # floor(6000*4096/10000) = 2457, floor(3999*4096/10000) = 1637, 200 -> max(1, 0) = 1: sum 4095,
        # the largest (3) takes the missing one
        want = {3: 2458, 9: 1637, 200: 1}
    blob = oracle.rns_encode(raw, raw.size)
    f, _, _ = _rns_region(blob, 64)
    assert {s: int(v) for s, v in enumerate(f) if v} == want
    assert np.array_equal(oracle.rns_decode(blob, raw.size), raw)


def test_rns_streams_interleave_and_emit_words():
    """Region byte j is symbol j div S of stream j mod S, and streams 64g .. 64g+63 share group g's
    words: a region where only stream 200 (group 3) carries information (every other byte 0)
    emits words in group 3 alone."""
    m = RNS_S * 40
    raw = np.zeros(m, np.uint8)
    rng = np.random.default_rng(2)
    raw[200::RNS_S] = rng.integers(1, 256, 40)
    blob = oracle.rns_encode(raw, m)
    f, states, offs = _rns_region(blob, 64)
    words = np.diff(offs.astype(np.int64))
    assert words[3] > 0 and words.sum() == words[3]
    assert np.array_equal(oracle.rns_decode(blob, m), raw)


def test_rns_group_words_in_lane_order():
    """Two streams of one group: 9 symbols each, alternating 1 and 2 in stream 0 and all 3 in
    stream 1, in a region of mostly 0 bytes (f[1] = f[2] = f[3] = 1 of 4096, so each of these
    symbols carries 12 bits and words are emitted at most steps; the other streams of
    the group hold only 0 bytes and emit none).  A decoder written here from the definition --
    symbols of the step for every stream, then the words in stream order -- reads the oracle's
    blob back to the bytes, ending on state 2^16 with every word of the group consumed."""
    m = RNS_S * 9
    raw = np.zeros(m, np.uint8)
    raw[0::RNS_S] = [1, 2] * 4 + [1]
    raw[1::RNS_S] = 3
    blob = oracle.rns_encode(raw, m)
    f, states, offs = _rns_region(blob, 64)
    assert offs[1] > 2  # group 0 emitted several words
    words = blob[64 + RNS_REGION_HEAD:64 + RNS_REGION_HEAD + 2 * int(offs[1])].view(np.uint16).astype(np.int64)
    c = np.concatenate([[0], np.cumsum(f.astype(np.int64))])
    x = [int(states[0]), int(states[1])]
    k, out = 0, [[], []]
    for j in range(9):
        for lane in (0, 1):
            slot = x[lane] & 4095
            sym = int(np.searchsorted(c, slot, side="right") - 1)
            out[lane].append(sym)
            x[lane] = int(f[sym]) * (x[lane] >> 12) + slot - int(c[sym])
        for lane in (0, 1):
            if x[lane] < 65536:
                x[lane] = (x[lane] << 16) | int(words[k])
                k += 1
    assert out[0] == [1, 2] * 4 + [1] and out[1] == [3] * 9
    assert x == [65536, 65536] and k == int(offs[1])


def test_rns_size_within_the_entropy_bound():
    """Independent bytes of a known distribution: every emitted word carries 16 bits of the code,
    so the words are at most the order-0 information of the symbols under the model's frequencies
    plus 16 bits per stream (the final state holds the rest)."""
    rng = np.random.default_rng(3)
    p = np.array([0.5, 0.25, 0.125, 0.0625, 0.0625])
    m = RNS_S * 64
    raw = rng.choice(5, m, p=p).astype(np.uint8)
    blob = oracle.rns_encode(raw, m)
    f, _, offs = _rns_region(blob, 64)
    info_bits = -np.log2(f[raw] / 4096.0).sum()
    words = int(offs[-1])
    assert 16 * words <= info_bits + 16 * RNS_S
    assert 16 * words >= info_bits - 32 * RNS_S
    assert np.array_equal(oracle.rns_decode(blob, m), raw)


@pytest.mark.parametrize("n,q", [(0, 0), (1, 0), (1, 1), (5000, 1234), (RNS_S * 3 + 7, RNS_S + 1)])
def test_rns_round_trip(n, q):
    rng = np.random.default_rng(n + q)
    raw = (rng.normal(0, 30, n).astype(np.int64) & 255).astype(np.uint8)
    blob = oracle.rns_encode(raw, q)
    assert np.array_equal(oracle.rns_decode(blob, n), raw)


def test_rns_decode_rejects_malformed_blobs():
    rng = np.random.default_rng(4)
    raw = rng.integers(0, 16, RNS_S * 40).astype(np.uint8)
    blob = oracle.rns_encode(raw, RNS_S * 20)
    words0 = int(_rns_region(blob, 64)[2][-1])
    second = 64 + (RNS_REGION_HEAD + 2 * words0 + 15) // 16 * 16
    # the magic, the size, a state and a word of region 0, the model of region 1
    for where in (0, 8, 64 + 512 + 4 * 3, 64 + RNS_REGION_HEAD + 2 * (words0 // 2), second + 2):
        bad = blob.copy()
        bad[where] ^= 0x5A
        with pytest.raises(ValueError):
            oracle.rns_decode(bad, raw.size)
    with pytest.raises(ValueError):
        oracle.rns_decode(blob[:1000], raw.size)
