"""GPU parity of the offloaded-bank path: LRU plans, fetched slot bytes and layer outputs against
the oracle, over several decode steps and layers with drifting expert popularity."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from synth import workloads as W  # noqa: E402

import mixture_experts_layer_token_amd as moe  # noqa: E402
from mixture_experts_layer_token_amd.layer import to_device_act  # noqa: E402
from mixture_experts_layer_token_amd.offload import OffloadedModel  # noqa: E402

from helpers import assert_output_close, say, to_f64  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


def run_and_check(wl, T, steps, check_steps, fill_all=True, capacity=None, policy="lru", period=0, overlap=True,
                  prefetch=None, pins=None, blob_bytes=None, work_slots=16, host_codec=None):
    """`blob_bytes`: compressed tiers with blob slots of that size (with `host_codec`: a bank of
    blobs of that codec in slots of that size, plain packages in HBM)."""
    tiers = blob_bytes is not None and host_codec is None
    xs = {}
    for s in range(steps):
        for l in range(wl.layers):
            x, _ = oracle.rank_gap_inputs(wl, T, layer=l, step=s)
            xs[(l, s)] = x
    model = OffloadedModel(wl, T, capacity=capacity, fill=fill_all, policy=policy, decay_period=period,
                           overlap=overlap, prefetch=prefetch, compressed=tiers,
                           blob_bytes=blob_bytes, work_slots=work_slots, host_codec=host_codec)
    if pins:
        model.reset_cache(pins=pins)
    if not fill_all:  # only the experts some step routes to (the others are never fetched)
        touched = {l: set() for l in range(wl.layers)}
        for (l, s), x in xs.items():
            lg = oracle.router_logits(wl.xdt, x, W.router_weights(wl, l), W.router_bias(wl, l, s))
            touched[l] |= set(oracle.topk_gates(lg, wl.k)[0].ravel().tolist())
        for l in range(wl.layers):
            model.fill(l, touched[l])
    groups, outs = [], {}
    for s in range(steps):
        for l in range(wl.layers):
            out = model.layer_forward(l, s, to_device_act(xs[(l, s)], wl.xdt))
            torch.cuda.synchronize()
            ids = model.layers[l].topk_ids[:T].cpu().numpy()
            groups.append((l * wl.E + ids.ravel()).tolist())
            if s in check_steps:
                outs[(l, s)] = to_f64(out)
                # what this layer's FFN read: every routed expert in the slot its table names, with the
                # bank's bytes; distinct experts in distinct slots
                tab = model.slot_tables[l].cpu().numpy()
                mine = sorted(set(ids.ravel().tolist()))
                slots = [int(tab[e]) for e in mine]
                assert min(slots) >= 0 and len(set(slots)) == len(slots)
                if host_codec:  # the slot holds the package the oracle decodes from the bank's blob
                    got_bytes = model.pool[torch.tensor(slots, device="cuda")][:, :model.raw_bytes].cpu().numpy()
                    # (full-size packages: six of the routed experts, spread over the list; the
                    # layer's outputs below cover every one of them)
                    pick = range(len(mine)) if model.raw_bytes < (4 << 20) else \
                        sorted(set(np.linspace(0, len(mine) - 1, min(6, len(mine))).astype(int).tolist()))
                    for i, e in ((i, mine[i]) for i in pick):
                        want = oracle.rns_decode(model.package(l, e)[:model.blob_sizes[l, e]], model.raw_bytes)
                        assert np.array_equal(got_bytes[i], want), ("decoded", l, s, e)
                else:
                    got_bytes = model.pool[torch.tensor(slots, device="cuda")][:, :model.pkg_bytes].cpu().numpy()
                    for i, e in enumerate(mine):
                        assert np.array_equal(got_bytes[i], model.package(l, e)), (l, s, e)
                if tiers:
                    # the working pool after the layer's last group: each of its experts' packages as the
                    # oracle decodes them from the blob
                    work = model.work[:len(model.last_group), :model.raw_bytes].cpu().numpy()
                    for i, e in enumerate(model.last_group):
                        want = oracle.xw4_decode(model.package(l, e), model.raw_bytes)
                        assert np.array_equal(work[i], want), ("decoded", l, s, e)
    # cache decisions: identical to the oracle's policy, over every demand lookup, prefetch and pin
    ev_groups = [(l * wl.E + np.asarray(ids)).tolist() for _, l, ids in model.events]
    kinds = [kind for kind, _, _ in model.events]
    h, m, v, ph = oracle.cache_sim(model.capacity, policy, period, ev_groups, kinds)
    dem = [i for i, kd in enumerate(kinds) if kd == "demand"]
    assert [(p[3], p[4]) for p in model.plans] == [(int(h[i]), int(m[i])) for i in dem]
    if prefetch is None and not pins:  # (then also the plain policy simulation)
        h0, m0, _ = (oracle.lru(model.capacity, groups) if policy == "lru"
                     else oracle.lfu_decay(model.capacity, period, groups))
        assert [(p[3], p[4]) for p in model.plans] == list(zip(h0.tolist(), m0.tolist()))
    st = model.cache.stats()
    assert st["hits"] == sum(h[i] for i in dem) and st["misses"] == sum(m[i] for i in dem)
    if host_codec:  # each fetch moved its blob's own bytes
        sizes = model.blob_sizes[model.blob_sizes > 0]
        assert m.sum() * sizes.min() <= st["bytes_fetched"] <= m.sum() * sizes.max()
        assert st["bytes_fetched"] % 16 == 0 and sizes.max() <= model.pkg_bytes
    else:
        assert st["bytes_fetched"] == m.sum() * model.pkg_bytes
    assert st["prefetch_hits"] == ph
    hb, _ = oracle.belady(model.capacity, groups)
    hd = sum(h[i] for i in dem)
    if prefetch is None and not pins:
        assert hb.sum() >= hd
    say("  %s prefetch %s pins %s: hits %d / %d lookups, prefetched %d, prefetch hits %d (belady %d)"
        % (policy, prefetch, bool(pins), hd, hd + sum(m[i] for i in dem), st["prefetch_fetches"], ph, hb.sum()))
    # outputs of the checked steps
    for (l, s), got_out in outs.items():
        experts = [None] * wl.E
        ids_ref, _ = oracle.topk_gates(oracle.router_logits(wl.xdt, xs[(l, s)], W.router_weights(wl, l),
                                                            W.router_bias(wl, l, s)), wl.k)
        for e in set(ids_ref.ravel().tolist()):
            experts[e] = W.expert_weights(wl, l, e)
        ref, ids, _ = oracle.moe_layer(wl.xdt, xs[(l, s)], W.router_weights(wl, l), W.router_bias(wl, l, s), wl.k,
                                       wl.I, experts)
        assert_output_close(got_out, ref, "bf16", "offload layer %d step %d" % (l, s))
    model.close()


@pytest.mark.parametrize("overlap", [True, False])
def test_offload_small_all_steps(overlap):
    """Every step checked; the FFN of the hits during the copies (two passes over the slot
    tables), or the whole FFN after them."""
    wl = W.Workload(name="offload-small", H=224, E=16, k=4, I=352, wfmt="int4g32", xdt="bf16", Ts=(5,), seed=606,
                    zipf_s=1.2, layers=3, steps=24, rerank_every=8, cache_frac=0.25)
    say("offload small, overlap", overlap)
    run_and_check(wl, 5, wl.steps, set(range(wl.steps)), overlap=overlap)


def test_offload_small_frequency_policy():
    wl = W.Workload(name="offload-lfu", H=224, E=16, k=4, I=352, wfmt="int4g32", xdt="bf16", Ts=(5,), seed=608,
                    zipf_s=1.2, layers=3, steps=24, rerank_every=8, cache_frac=0.25)
    say("offload small, lfu-decay")
    run_and_check(wl, 5, wl.steps, {0, 11, 23}, policy="lfu_decay", period=6)


@pytest.mark.parametrize("prefetch,policy", [("last", "lru"), ("popular", "lfu_decay")])
def test_offload_small_prefetch(prefetch, policy):
    """Fetching the next layer's likely experts while a layer computes: every step checked (outputs,
    slot bytes), every lookup, prefetch and eviction against the oracle's simulation."""
    wl = W.Workload(name="offload-pf", H=224, E=16, k=4, I=352, wfmt="int4g32", xdt="bf16", Ts=(5,), seed=609,
                    zipf_s=1.2, layers=3, steps=24, rerank_every=8, cache_frac=0.4)
    say("offload small, prefetch", prefetch, policy)
    run_and_check(wl, 5, wl.steps, set(range(wl.steps)), policy=policy, period=6 if policy != "lru" else 0,
                  prefetch=prefetch)


def test_offload_small_static_pin():
    """Two experts of every layer pinned for the whole run, LRU over the other slots."""
    wl = W.Workload(name="offload-pin", H=224, E=16, k=4, I=352, wfmt="int4g32", xdt="bf16", Ts=(5,), seed=610,
                    zipf_s=1.2, layers=3, steps=20, rerank_every=8, cache_frac=0.4)
    say("offload small, static pin")
    run_and_check(wl, 5, wl.steps, {0, 9, 19}, pins={l: [l, l + 5] for l in range(wl.layers)})


def test_offload_small_tight_capacity():
    wl = W.Workload(name="offload-tight", H=96, E=32, k=8, I=160, wfmt="mxfp4", xdt="bf16", Ts=(3,), seed=607,
                    zipf_s=0.8, layers=2, steps=16, rerank_every=4, cache_frac=0.25)
    say("offload tight")
    run_and_check(wl, 3, wl.steps, {0, 7, 15}, capacity=24)


@pytest.mark.parametrize("T,prefetch", [(1, None), (16, None), (16, "last")])
def test_offload_glm_full_size_first_steps(T, prefetch):
    """GLM-shaped layers at full size (bank filled with every expert the first steps route to)."""
    wl = W.WORKLOADS["glm"].with_(steps=3)
    say("offload glm full size T", T, "prefetch", prefetch)
    run_and_check(wl, T, 3, {0, 2}, fill_all=False, prefetch=prefetch)


@pytest.mark.parametrize("overlap,work_slots", [(True, 16), (False, 16), (True, 3), (False, 1)])
def test_offload_compressed_small_all_steps(overlap, work_slots):
    """bf16 experts in compressed tiers: blobs in the bank and in the HBM slots, decoded into the
    working pool in groups of at most `work_slots` experts, each followed by its FFN pass; every
    step checked (slot bytes, decoded packages, outputs)."""
    from mixture_experts_layer_token_amd import api

    wl = W.Workload(name="offload-z", H=224, E=16, k=4, I=352, wfmt="bf16", xdt="bf16", Ts=(5,), seed=611,
                    zipf_s=1.2, layers=3, steps=16, rerank_every=8, cache_frac=0.25)
    blob = (api.moe_compress_bound(api.moe_package_bytes(wl.H, wl.I, "bf16")) + 255) // 256 * 256
    say("offload compressed small, overlap", overlap, "work slots", work_slots)
    run_and_check(wl, 5, wl.steps, set(range(wl.steps)), overlap=overlap, blob_bytes=blob, work_slots=work_slots)


def test_offload_compressed_glm_bf16_full_size_first_steps():
    """GLM-shaped bf16 experts at full size (two layers), compressed tiers with blob slots of 77% of
    the package, frequency-with-decay policy."""
    from mixture_experts_layer_token_amd import api

    wl = W.WORKLOADS["glm"].with_(wfmt="bf16", layers=2, steps=3, name="glm-bf16")
    raw = api.moe_package_bytes(wl.H, wl.I, "bf16")
    blob = (int(raw * 0.77) + 255) // 256 * 256
    say("offload compressed glm bf16")
    run_and_check(wl, 4, 3, {0, 2}, fill_all=False, policy="lfu_decay", period=4, blob_bytes=blob)


@pytest.mark.parametrize("overlap,prefetch,fmt", [(True, None, "int4g32"), (False, "last", "mxfp4")])
def test_offload_rans_bank_small_all_steps(overlap, prefetch, fmt):
    """4-bit experts with a bank of rANS blobs: every miss decoded into its plain HBM slot on the
    cache's decode stream; every step checked (slot bytes against the oracle's decode, outputs)."""
    from mixture_experts_layer_token_amd import api

    wl = W.Workload(name="offload-r", H=224, E=16, k=4, I=352, wfmt=fmt, xdt="bf16", Ts=(5,), seed=612,
                    zipf_s=1.2, layers=3, steps=16, rerank_every=8, cache_frac=0.3)
    blob = (api.moe_compress_rans_bound(api.moe_package_bytes(wl.H, wl.I, fmt)) + 255) // 256 * 256
    say("offload rans bank small", fmt, "overlap", overlap, "prefetch", prefetch)
    run_and_check(wl, 5, wl.steps, set(range(wl.steps)), overlap=overlap, prefetch=prefetch, blob_bytes=blob,
                  host_codec="rans")


@pytest.mark.parametrize("T", [1, 16])
def test_offload_rans_bank_glm_full_size_first_steps(T):
    """GLM-shaped INT4 layers at full size with a bank of rANS blobs in slots of 90% of the package."""
    from mixture_experts_layer_token_amd import api

    wl = W.WORKLOADS["glm"].with_(layers=2, steps=3)
    raw = api.moe_package_bytes(wl.H, wl.I, wl.wfmt)
    blob = (int(raw * 0.9) + 255) // 256 * 256
    say("offload rans bank glm T", T)
    run_and_check(wl, T, 3, {0, 2}, fill_all=False, blob_bytes=blob, host_codec="rans")


@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_slots_outside_the_pool_are_skipped(mode):
    """Experts whose slot-table entry is -1 or past the pool are skipped (rows left as they were);
    resident experts are computed from the slot their entry names."""
    from mixture_experts_layer_token_amd import api

    from helpers import small_variant

    wl = small_variant("int4g32", E=4, k=1, name="slot-guard")
    T = 96 if mode == "prefill" else 8
    nb = api.moe_package_bytes(wl.H, wl.I, wl.wfmt)
    stride = (nb + 255) // 256 * 256
    ex = [W.expert_weights(wl, 0, e) for e in range(4)]
    pool = torch.zeros((2, stride), dtype=torch.uint8, device="cuda")
    pool[0, :nb] = torch.from_numpy(api.moe_pack_expert(wl.H, wl.I, wl.wfmt, ex[2]))  # expert 2 -> slot 0
    pool[1, :nb] = torch.from_numpy(api.moe_pack_expert(wl.H, wl.I, wl.wfmt, ex[0]))  # expert 0 -> slot 1
    table = torch.tensor([1, -1, 0, 7], dtype=torch.int32, device="cuda")
    desc = api.experts_desc(wl.H, wl.I, 4, wl.wfmt, pool, stride, table)
    assert desc.n_slots == 2
    ids = torch.tensor([[t % 4] for t in range(T)], dtype=torch.int32, device="cuda")
    counts = torch.empty(4, dtype=torch.int32, device="cuda")
    offsets = torch.empty(5, dtype=torch.int32, device="cuda")
    perm = torch.empty(T, dtype=torch.int32, device="cuda")
    inv = torch.empty(T, dtype=torch.int32, device="cuda")
    api.moe_permute(ids, 4, counts, offsets, perm, inv)
    x_host = W.activations(wl, T)
    x = to_device_act(x_host, "bf16")
    y = torch.full((T, wl.H), 12345.0, dtype=torch.float32, device="cuda")
    ws = torch.empty(api.moe_ffn_workspace(desc, T, 1), dtype=torch.uint8, device="cuda")
    api.moe_expert_ffn(desc, x, 1, offsets, perm, y, ws, mode=mode)
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    o = offsets.cpu().numpy()
    xd = oracle.decode_act("bf16", x_host)
    for e in range(4):
        rows = perm.cpu().numpy()[o[e]:o[e + 1]]
        got = yh[o[e]:o[e + 1]]
        if e in (1, 3):
            assert np.all(got == 12345.0)
        else:
            ref = oracle.ffn(ex[e], wl.H, wl.I, xd[rows])
            assert_output_close(got.astype(np.float64), ref, "bf16", "slot guard expert %d" % e)


@pytest.mark.parametrize("T", [1, 16])
def test_glm_full_run_planner_vs_oracle(T):
    """The whole lookup sequence of the GLM-shaped offload run (256 steps x 8 layers, the activations
    the offload bench routes, no rank-gap redraw): routed on the GPU, planned by the library's
    planner under both policies the bench reports, and compared group by group with the oracle's
    LRU and frequency-with-decay simulations (hits, misses) and the Belady bound."""
    from mixture_experts_layer_token_amd import api
    from mixture_experts_layer_token_amd.api import ExpertCache

    wl = W.WORKLOADS["glm"]
    say("glm planner, T", T)
    ids = torch.empty((T, wl.k), dtype=torch.int32, device="cuda")
    gw = torch.empty((T, wl.k), dtype=torch.float32, device="cuda")
    wg = [to_device_act(W.router_weights(wl, l), wl.xdt) for l in range(wl.layers)]
    bias = {}
    groups = []
    for s in range(wl.steps):
        for l in range(wl.layers):
            ep = s // wl.rerank_every
            if (l, ep) not in bias:
                bias[(l, ep)] = torch.from_numpy(W.router_bias(wl, l, s)).cuda()
            x = to_device_act(W.activations(wl, T, l, s), wl.xdt)
            api.moe_route(x, wg[l], bias[(l, ep)], wl.k, ids, gw)
            got = ids.cpu().numpy()
            assert got.min() >= 0 and got.max() < wl.E
            assert all(len(set(r.tolist())) == wl.k for r in got)
            groups.append((l * wl.E + got.ravel()).tolist())
    cap = int(wl.cache_frac * wl.layers * wl.E)
    for policy, period in (("lru", 0), ("lfu_decay", 32)):
        c = ExpertCache(None, 1 << 20, wl.layers, wl.E, None, 0, cap, policy, period)
        plans = [c.plan(g % wl.layers, np.array(grp, dtype=np.int64) - (g % wl.layers) * wl.E)
                 for g, grp in enumerate(groups)]
        if policy == "lru":
            h, m, _ = oracle.lru(cap, groups)
        else:
            h, m, _ = oracle.lfu_decay(cap, period, groups)
        assert [p.n_hits for p in plans] == h.tolist()
        assert [p.n_misses for p in plans] == m.tolist()
        hb, _ = oracle.belady(cap, groups)
        assert hb.sum() >= h.sum()
        say("  %s: hit rate %.4f (belady %.4f) over %d lookups" % (policy, h.sum() / (h.sum() + m.sum()),
                                                                  hb.sum() / (h.sum() + m.sum()), h.sum() + m.sum()))
        c.close()
