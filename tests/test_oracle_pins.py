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
