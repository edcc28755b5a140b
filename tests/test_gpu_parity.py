"""GPU parity: the HIP path through the C-ABI against the fp64 oracle.

Integer results (routing ids, permutation) and dequantized weights are compared
bit-exactly; gate weights to 1e-5 relative (a gate's relative error is at most
twice the largest logit error, and fp32 accumulation of H <= 8192 exact products
leaves logit errors near 1e-6); layer outputs to rel-L2 <= 5e-3 and max-abs <=
2e-2 * max|ref| (bf16 activations) or rel-L2 <= 1e-5 (fp32).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from synth import workloads as W  # noqa: E402

import mixture_experts_layer_token_amd as moe  # noqa: E402
from mixture_experts_layer_token_amd.layer import build_layer, to_device_act  # noqa: E402

from helpers import assert_output_close, oracle_reference, say, small_variant, to_f64  # noqa: E402


GATE_RTOL, GATE_ATOL = 1e-5, 1e-6


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


# ------------------------------------------------------------------ dequant

@pytest.mark.parametrize("fmt", ["f32", "bf16", "mxfp4", "int4g32"])
@pytest.mark.parametrize("H,I", [(224, 352), (2880, 96), (64, 2880)])
def test_dequant_bit_exact(fmt, H, I):
    say("dequant", fmt, H, I)
    wl = small_variant(fmt, H=H, I=I, name="dq-%s-%d-%d" % (fmt, H, I))
    ex = W.expert_weights(wl, 0, 5)
    pkg = moe.moe_pack_expert(H, I, fmt, ex)
    d_pkg = torch.from_numpy(pkg).cuda()
    out = torch.empty(3 * H * I, dtype=torch.float32, device="cuda")
    moe.moe_dequant_expert(d_pkg, H, I, fmt, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = np.concatenate([oracle.decode(fmt, ex["w"][m], ex["s"][m], *shp).ravel()
                           for m, shp in enumerate([(I, H), (I, H), (H, I)])]).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def _sweep_scales_int4(n):
    """bf16 scales that binary16 holds exactly (the packer's domain) and whose products with every
    code stay finite in binary16 (8 * s <= 65504): 2^-14 .. 2^12 with a spread of 8-bit mantissas,
    zero and a negative value."""
    vals = []
    for ex in range(-14, 13):
        for m in range(0, 128, 9):
            vals.append(np.float32(2.0 ** ex * (1 + m / 128.0)))
    vals += [np.float32(0.0), np.float32(-0.75)]
    v = np.array(vals, np.float32).view(np.uint32) >> 16
    return np.resize(v.astype(np.uint16), n)


@pytest.mark.parametrize("fmt", ["mxfp4", "int4g32"])
def test_dequant_every_code_and_scale(fmt):
    """All 256 code bytes against every E8M0 exponent whose products stay finite in fp32 (0..252)
    plus the NaN scale 0xFF, or a sweep of binary16-exact INT4 scales: the in-register decoders
    the FFN kernels use."""
    H, I = 256, 320
    say("dequant sweep", fmt)
    rng = np.random.default_rng(77)
    ex = {"w": [], "s": []}
    for rows, K in ((I, H), (I, H), (H, I)):
        codes = rng.permutation(np.resize(np.arange(256, dtype=np.uint8), rows * K // 2)).reshape(rows, K // 2)
        ng = rows * K // 32
        if fmt == "mxfp4":
            sc = np.resize(np.append(np.arange(253, dtype=np.uint8), np.uint8(255)), ng)
        else:
            sc = _sweep_scales_int4(ng)
        ex["w"].append(codes)
        ex["s"].append(rng.permutation(sc).reshape(rows, K // 32))
    pkg = moe.moe_pack_expert(H, I, fmt, ex)
    out = torch.empty(3 * H * I, dtype=torch.float32, device="cuda")
    moe.moe_dequant_expert(torch.from_numpy(pkg).cuda(), H, I, fmt, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = np.concatenate([oracle.decode(fmt, ex["w"][m], ex["s"][m], *shp).ravel()
                           for m, shp in enumerate([(I, H), (I, H), (H, I)])]).astype(np.float32)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


# ------------------------------------------------------------------ router

ROUTE_CASES = [
    ("tiny", 16, {}),
    ("mixtral", 64, {}),
    ("gptoss", 512, {}),
    ("kimi", 300, {}),
    ("tiny", 16, dict(E=1, k=1, name="e1k1")),
    ("tiny", 16, dict(k=8, name="k-eq-e")),
    ("tiny", 37, dict(E=1024, k=16, H=64, name="e1024", xdt="bf16")),
    ("tiny", 300, dict(E=24, k=3, name="e24-bf16", xdt="bf16")),  # large T, E not a multiple of 16
    ("tiny", 700, dict(E=48, k=5, H=96, name="e48-bf16", xdt="bf16")),  # large T, ragged row tile
    # T * E > 2^20: the MFMA tile kernel in short row tiles (the last one ragged), two column tiles
    ("tiny", 3000, dict(E=400, k=6, H=96, name="e400-bf16-tile", xdt="bf16")),
    # T * E > 2^20 with E not a multiple of 16: the one-kernel bf16 router (16 tokens per workgroup)
    ("tiny", 50000, dict(E=24, k=3, H=96, name="e24-bf16-onekernel", xdt="bf16")),
]


@pytest.mark.parametrize("name,T,kw", ROUTE_CASES, ids=[c[0] + "-" + str(c[1]) + str(c[2].get("name", ""))
                                                         for c in ROUTE_CASES])
def test_route_exact(name, T, kw):
    wl = W.WORKLOADS[name].with_(**kw)
    say("route", wl.name, "T", T, "E", wl.E, "k", wl.k)
    x, _ = oracle.rank_gap_inputs(wl, T)
    wg = W.router_weights(wl)
    bias = W.router_bias(wl)
    lg = oracle.router_logits(wl.xdt, x, wg, bias)
    ids_ref, w_ref = oracle.topk_gates(lg, wl.k)
    xd, wgd = to_device_act(x, wl.xdt), to_device_act(wg, wl.xdt)
    bd = torch.from_numpy(bias).cuda() if bias is not None else None
    ids = torch.empty((T, wl.k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, wl.k), dtype=torch.float32, device="cuda")
    logits = torch.empty((T, wl.E), dtype=torch.float32, device="cuda")
    moe.moe_route(xd, wgd, bd, wl.k, ids, w, logits)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    np.testing.assert_allclose(w.cpu().numpy(), w_ref, rtol=GATE_RTOL, atol=GATE_ATOL)
    # a token's gates sum to one up to fp32 rounding: k exponentials of relative error <= 2^-23,
    # their fp32 sum (<= (k - 1) roundings of 2^-24) and one division (2^-24) per gate
    wsum = w.cpu().numpy().astype(np.float64).sum(axis=1)
    assert np.abs(wsum - 1.0).max() <= (wl.k + 3) * 2.0 ** -23, np.abs(wsum - 1.0).max()
    np.testing.assert_allclose(logits.cpu().numpy(), lg, rtol=1e-4, atol=1e-4 * np.abs(lg).max())


# router inputs that are not finite: the ids stay distinct and in [0, E) on every router path
ROUTE_NAN_CASES = [
    ("tiny", 16, {}),                                                       # fp32, one workgroup per token
    ("tiny", 300, dict(E=24, k=3, name="nan-split", xdt="bf16")),           # split over workgroups
    ("tiny", 50000, dict(E=24, k=3, H=96, name="nan-onekernel", xdt="bf16")),  # one-kernel bf16 router
    ("tiny", 3000, dict(E=400, k=6, H=96, name="nan-tile", xdt="bf16")),    # MFMA tile kernel
]


def _poison(x, xdt, rows):
    """x with row rows[0] all NaN, row rows[1] holding one +inf and row rows[2] one NaN element."""
    x = x.copy()
    nan, inf = (np.float32(np.nan), np.float32(np.inf)) if xdt == "f32" else (np.uint16(0x7FC0), np.uint16(0x7F80))
    x[rows[0], :] = nan
    x[rows[1], 5] = inf
    x[rows[2], 3] = nan
    return x


@pytest.mark.parametrize("name,T,kw", ROUTE_NAN_CASES, ids=[c[2].get("name", c[0]) for c in ROUTE_NAN_CASES])
def test_route_nonfinite_rows(name, T, kw):
    """A token whose logits are NaN or infinite gets k distinct ids in [0, E) (infinite and finite
    logits first, NaN last, equal keys to the lower id: an all-NaN row takes ids 0..k-1); every other
    token's routing is unchanged."""
    wl = W.WORKLOADS[name].with_(**kw)
    say("route non-finite rows", wl.name, "T", T)
    x, _ = oracle.rank_gap_inputs(wl, T)
    bad = [1, T // 2, T - 1]
    xp = _poison(x, wl.xdt, bad)
    wg, bias = W.router_weights(wl), W.router_bias(wl)
    ids_ref, _ = oracle.topk_gates(oracle.router_logits(wl.xdt, x, wg, bias), wl.k)
    ids = torch.empty((T, wl.k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, wl.k), dtype=torch.float32, device="cuda")
    bd = torch.from_numpy(bias).cuda() if bias is not None else None
    moe.moe_route(to_device_act(xp, wl.xdt), to_device_act(wg, wl.xdt), bd, wl.k, ids, w)
    torch.cuda.synchronize()
    got = ids.cpu().numpy()
    assert got.min() >= 0 and got.max() < wl.E
    assert all(len(set(r.tolist())) == wl.k for r in got)
    assert got[bad[0]].tolist() == list(range(wl.k))
    good = np.setdiff1d(np.arange(T), bad)
    assert np.array_equal(got[good], ids_ref[good])
    assert np.isnan(w.cpu().numpy()[bad[0]]).all()


@pytest.mark.parametrize("fmt", ["bf16", "mxfp4", "int4g32"])
@pytest.mark.parametrize("mode", ["auto", "prefill"])
def test_layer_nonfinite_token_leaves_others_exact(fmt, mode):
    """One all-NaN token and one token with an infinite element go through the whole layer: every
    other token's routing and output match the oracle."""
    wl = small_variant(fmt)
    T = 40
    say("layer non-finite tokens", wl.name, mode)
    x, _ = oracle.rank_gap_inputs(wl, T)
    bad = [3, 20, 37]
    layer = build_layer(wl, T)
    out = layer.forward(to_device_act(_poison(x, wl.xdt, bad), wl.xdt), mode=mode)
    torch.cuda.synchronize()
    ids = layer.topk_ids[:T].cpu().numpy()
    assert ids.min() >= 0 and ids.max() < wl.E
    good = np.setdiff1d(np.arange(T), bad)
    ref, ids_ref, _ = oracle_reference(wl, x, good)
    assert np.array_equal(ids[good], ids_ref)
    assert_output_close(to_f64(out)[good], ref, "bf16", wl.name + " finite tokens")


# ------------------------------------------------------------------ permutation

PERM_CASES = [(0, 2, 8), (1, 1, 1), (16, 2, 8), (64, 2, 8), (512, 4, 128), (8192, 8, 384), (100, 16, 1024),
              (333, 3, 7), (4096, 16, 1024), (1025, 8, 16), (2048, 4, 5)]


@pytest.mark.parametrize("T,k,E", PERM_CASES)
def test_permute_exact(T, k, E):
    say("permute", T, k, E)
    rng = np.random.default_rng(T * 7 + k * 3 + E)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32) if T else np.zeros((0, k), np.int32)
    if T > 10:
        ids[: T // 3, 0] = 0  # a hot expert
    c_ref, o_ref, p_ref, i_ref = oracle.permute(ids, E)
    d_ids = torch.from_numpy(ids).cuda()
    n = max(T * k, 1)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(n, dtype=torch.int32, device="cuda")
    inv = torch.empty(n, dtype=torch.int32, device="cuda")
    moe.moe_permute(d_ids, E, counts, offsets, perm, inv)
    torch.cuda.synchronize()
    assert np.array_equal(counts.cpu().numpy(), c_ref)
    assert np.array_equal(offsets.cpu().numpy(), o_ref)
    assert np.array_equal(perm.cpu().numpy()[:T * k], p_ref)
    assert np.array_equal(inv.cpu().numpy()[:T * k], i_ref)


def test_permute_all_tokens_one_expert():
    T, k, E = 1000, 1, 16
    ids = np.full((T, k), 11, dtype=np.int32)
    d_ids = torch.from_numpy(ids).cuda()
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(T, dtype=torch.int32, device="cuda")
    inv = torch.empty(T, dtype=torch.int32, device="cuda")
    moe.moe_permute(d_ids, E, counts, offsets, perm, inv)
    torch.cuda.synchronize()
    assert counts.cpu().numpy()[11] == T and np.array_equal(perm.cpu().numpy(), np.arange(T))


# ------------------------------------------------------------------ router + permutation in one call

# (workload, T, overrides, poisoned rows): decode batches on the one-workgroup path (T <= 16,
# T*k <= 1024), the largest rows it takes (E = 1024 with k = 16), and batches beyond it
ROUTE_PERMUTE_CASES = [
    ("gptoss", 1, {}, ()), ("gptoss", 3, {}, ()), ("gptoss", 16, {}, ()), ("gptoss", 17, {}, ()),
    ("gptoss", 64, {}, ()), ("mixtral", 16, {}, ()), ("kimi", 1, {}, ()), ("kimi", 16, {}, ()),
    ("kimi", 128, {}, ()), ("glm", 16, {}, ()),
    ("tiny", 16, dict(E=1024, k=16, H=64, name="e1024k16", xdt="bf16"), ()),
    ("tiny", 17, dict(E=1024, k=16, H=64, name="e1024k16", xdt="bf16"), ()),
    ("tiny", 7, dict(E=1, k=1, name="e1k1", xdt="bf16"), ()),
    ("tiny", 16, {}, ()),  # fp32 activations: the two calls' kernels
    ("tiny", 0, dict(xdt="bf16", name="empty"), ()),
    ("gptoss", 12, dict(name="nonfinite"), (1, 6, 11)),
    ("gptoss", 40, dict(name="nonfinite"), (1, 20, 39)),
]


@pytest.mark.parametrize("name,T,kw,bad", ROUTE_PERMUTE_CASES,
                         ids=["%s-%d%s" % (c[0], c[1], c[2].get("name", "")) for c in ROUTE_PERMUTE_CASES])
def test_route_permute_exact(name, T, kw, bad):
    """moe_route_permute: ids and grouping equal the oracle's, bit for bit; ids, gates, logits and
    grouping equal those of moe_route followed by moe_permute, bit for bit."""
    wl = W.WORKLOADS[name].with_(**kw)
    k, E = wl.k, wl.E
    say("route+permute", wl.name, "T", T, "E", E, "k", k, wl.xdt)
    if T:
        x, _ = oracle.rank_gap_inputs(wl, T)
    else:
        x = np.zeros((0, wl.H), np.float32 if wl.xdt == "f32" else np.uint16)
    if bad:
        x = _poison(x, wl.xdt, list(bad))
    wg, bias = W.router_weights(wl), W.router_bias(wl)
    xd, wgd = to_device_act(x, wl.xdt), to_device_act(wg, wl.xdt)
    bd = torch.from_numpy(bias).cuda() if bias is not None else None
    n = max(T * k, 1)

    def outs():
        i32 = dict(dtype=torch.int32, device="cuda")
        return (torch.full((T, k), -7, **i32), torch.full((T, k), -7.0, device="cuda"),
                torch.full((T, E), -7.0, device="cuda"), torch.full((E,), -7, **i32),
                torch.full((E + 1,), -7, **i32), torch.full((n,), -7, **i32), torch.full((n,), -7, **i32))

    ids, w, lg, counts, offsets, perm, inv = a = outs()
    moe.moe_route_permute(xd, wgd, bd, k, ids, w, counts, offsets, perm, inv, logits=lg)
    ids2, w2, lg2, counts2, offsets2, perm2, inv2 = b = outs()
    moe.moe_route(xd, wgd, bd, k, ids2, w2, lg2)
    moe.moe_permute(ids2, E, counts2, offsets2, perm2, inv2)
    torch.cuda.synchronize()
    for u, v, what in zip(a, b, ("ids", "gates", "logits", "counts", "offsets", "perm", "inv")):
        un, vn = u.cpu().numpy(), v.cpu().numpy()
        if u.dtype == torch.float32:
            un, vn = un.view(np.uint32), vn.view(np.uint32)  # bit patterns (NaN included)
        if what in ("perm", "inv"):
            un, vn = un[:T * k], vn[:T * k]
        assert np.array_equal(un, vn), what
    got = ids.cpu().numpy()
    c_ref, o_ref, p_ref, i_ref = oracle.permute(got, E)
    assert np.array_equal(counts.cpu().numpy(), c_ref)
    assert np.array_equal(offsets.cpu().numpy(), o_ref)
    assert np.array_equal(perm.cpu().numpy()[:T * k], p_ref)
    assert np.array_equal(inv.cpu().numpy()[:T * k], i_ref)
    if T == 0:
        return
    good = np.setdiff1d(np.arange(T), np.asarray(bad, np.int64))
    lgr = oracle.router_logits(wl.xdt, x[good], wg, bias)
    ids_ref, w_ref = oracle.topk_gates(lgr, k)
    assert np.array_equal(got[good], ids_ref)
    np.testing.assert_allclose(w.cpu().numpy()[good], w_ref, rtol=GATE_RTOL, atol=GATE_ATOL)
    if bad:
        assert got.min() >= 0 and got.max() < E and all(len(set(r.tolist())) == k for r in got)
        assert got[bad[0]].tolist() == list(range(k))


# ------------------------------------------------------------------ whole layer, reduced shapes

SMALL = [("f32", "f32"), ("f32", "bf16"), ("bf16", "bf16"), ("mxfp4", "bf16"), ("int4g32", "bf16"),
         ("bf16", "f32"), ("int4g32", "f32")]


@pytest.mark.parametrize("fmt,xdt", SMALL)
@pytest.mark.parametrize("T", [1, 3, 40, 130])
@pytest.mark.parametrize("mode", ["auto", "decode", "prefill"])
def test_layer_small(fmt, xdt, T, mode):
    if fmt == "f32" and mode != "auto":
        pytest.skip("fp32 experts have one (VALU) variant")
    wl = small_variant(fmt, xdt)
    say("layer small", wl.name, "T", T, "mode", mode)
    x, _ = oracle.rank_gap_inputs(wl, T)
    layer = build_layer(wl, T)
    out = layer.forward(to_device_act(x, xdt), mode=mode)
    torch.cuda.synchronize()
    ref, ids_ref, w_ref = oracle_reference(wl, x, np.arange(T))
    assert np.array_equal(layer.topk_ids[:T].cpu().numpy(), ids_ref)
    np.testing.assert_allclose(layer.topk_w[:T].cpu().numpy(), w_ref, rtol=GATE_RTOL, atol=GATE_ATOL)
    tol_dt = "f32" if (fmt == "f32" and xdt == "f32") else "bf16"
    assert_output_close(to_f64(out), ref, tol_dt, wl.name)


@pytest.mark.parametrize("fmt,xdt", [("f32", "f32"), ("bf16", "bf16"), ("mxfp4", "bf16"), ("int4g32", "bf16")])
@pytest.mark.parametrize("mode", ["auto", "decode", "prefill"])
def test_layer_empty_batch_then_batch(fmt, xdt, mode):
    """T = 0: every call of the path succeeds and does nothing; the same layer then computes a
    ragged batch correctly (the workspaces and plans of the empty call leave nothing behind)."""
    if fmt == "f32" and mode != "auto":
        pytest.skip("fp32 experts have one (VALU) variant")
    wl = small_variant(fmt, xdt)
    say("layer empty batch", wl.name, "mode", mode)
    layer = build_layer(wl, 8)
    x0 = np.zeros((0, wl.H), np.float32 if xdt == "f32" else np.uint16)
    out0 = layer.forward(to_device_act(x0, xdt), mode=mode)
    torch.cuda.synchronize()
    assert tuple(out0.shape) == (0, wl.H)
    x, _ = oracle.rank_gap_inputs(wl, 5)
    out = layer.forward(to_device_act(x, xdt), mode=mode)
    torch.cuda.synchronize()
    ref, ids_ref, _ = oracle_reference(wl, x, np.arange(5))
    assert np.array_equal(layer.topk_ids[:5].cpu().numpy(), ids_ref)
    assert_output_close(to_f64(out), ref, "f32" if fmt == "f32" else "bf16", wl.name)


@pytest.mark.parametrize("fmt", ["bf16", "mxfp4", "int4g32"])
def test_layer_hot_expert_split(fmt):
    """Skewed routing: a few experts get hundreds of rows (MFMA tile kernel), the rest a handful
    (streaming kernel), in one call.  (bf16: 64 experts, top-2, so that the average stays below
    the 28 rows per expert from which every bf16 expert goes to the tile kernel.)"""
    kw = dict(E=64, k=2, zipf_s=0.8) if fmt == "bf16" else dict(zipf_s=3.0)
    wl = small_variant(fmt, name="hot-" + fmt, **kw)
    T = 300
    say("hot expert split", wl.name)
    x, _ = oracle.rank_gap_inputs(wl, T)
    layer = build_layer(wl, T)
    out = layer.forward(to_device_act(x, "bf16"))
    torch.cuda.synchronize()
    counts = layer.counts.cpu().numpy()
    assert counts.max() > 128 and 0 < counts[counts > 0].min() <= 128  # both variants have work
    ref, ids_ref, _ = oracle_reference(wl, x, np.arange(T))
    assert np.array_equal(layer.topk_ids[:T].cpu().numpy(), ids_ref)
    assert_output_close(to_f64(out), ref, "bf16", wl.name)


@pytest.mark.parametrize("fmt", ["bf16", "mxfp4", "int4g32"])
@pytest.mark.parametrize("mode", ["auto", "prefill"])
def test_layer_max_experts_and_top_k(fmt, mode):
    """The largest routing the boundary accepts: E = 1024 experts, top-16, on narrow experts, so
    that every kernel sees 1024 row groups (most of them empty) and the combine sums 16 rows."""
    wl = small_variant(fmt, E=1024, k=16, H=64, I=96, name="maxek-" + fmt)
    T = 48
    say("layer E=1024 k=16", wl.name, "mode", mode)
    x, _ = oracle.rank_gap_inputs(wl, T)
    layer = build_layer(wl, T)
    out = layer.forward(to_device_act(x, "bf16"), mode=mode)
    torch.cuda.synchronize()
    ref, ids_ref, w_ref = oracle_reference(wl, x, np.arange(T))
    assert np.array_equal(layer.topk_ids[:T].cpu().numpy(), ids_ref)
    np.testing.assert_allclose(layer.topk_w[:T].cpu().numpy(), w_ref, rtol=GATE_RTOL, atol=GATE_ATOL)
    assert_output_close(to_f64(out), ref, "bf16", wl.name)


@pytest.mark.parametrize("fmt", ["mxfp4", "int4g32"])
@pytest.mark.parametrize("T", [64, 200])
def test_layer_many_experts_4bit(fmt, T):
    """Many experts touched (E = 128, top-8) at small H and I with ragged 4-bit chunks: the streaming
    kernel with activations shared through LDS, at one (T = 64) and two (T = 200) M tiles."""
    wl = small_variant(fmt, E=128, k=8, name="wide-" + fmt)
    say("many experts", wl.name, "T", T)
    x, _ = oracle.rank_gap_inputs(wl, T)
    layer = build_layer(wl, T)
    out = layer.forward(to_device_act(x, "bf16"), mode="decode")
    torch.cuda.synchronize()
    assert (layer.counts.cpu().numpy() > 0).sum() > 64  # wide: most experts have rows
    ref, ids_ref, _ = oracle_reference(wl, x, np.arange(T))
    assert np.array_equal(layer.topk_ids[:T].cpu().numpy(), ids_ref)
    assert_output_close(to_f64(out), ref, "bf16", wl.name)


def test_tiny_config_full():
    wl = W.WORKLOADS["tiny"]
    T = wl.Ts[0]
    say("tiny config", T)
    x, _ = oracle.rank_gap_inputs(wl, T)
    layer = build_layer(wl, T)
    out = layer.forward(to_device_act(x, wl.xdt))
    torch.cuda.synchronize()
    ref, ids_ref, _ = oracle_reference(wl, x, np.arange(T))
    assert np.array_equal(layer.topk_ids.cpu().numpy(), ids_ref)
    assert_output_close(to_f64(out), ref, "f32", "tiny")


def test_layer_deterministic():
    wl = small_variant("mxfp4")
    x, _ = oracle.rank_gap_inputs(wl, 40)
    layer = build_layer(wl, 40)
    xd = to_device_act(x, "bf16")
    a = layer.forward(xd).clone()
    b = layer.forward(xd).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_shared_expert_small():
    wl = small_variant("int4g32", shared=True, name="small-shared")
    T = 40
    say("shared expert", wl.name)
    x, _ = oracle.rank_gap_inputs(wl, T)
    layer = build_layer(wl, T)
    out = layer.forward(to_device_act(x, "bf16"))
    torch.cuda.synchronize()
    ref, _, _ = oracle_reference(wl, x, np.arange(T))
    assert_output_close(to_f64(out), ref, "bf16", wl.name)


@pytest.mark.parametrize("sigma,xdt", [(1e-3, "bf16"), (100.0, "bf16"), (3e4, "bf16"), (3e4, "f32")])
@pytest.mark.parametrize("mode", ["auto", "decode", "prefill"])
def test_int4_activation_magnitudes(sigma, xdt, mode):
    """INT4 experts run on binary16 operands.  Kimi-wide rows (H = 7168) with N(0, sigma)
    activations: at sigma = 3e4 the activations themselves exceed binary16's range, at sigma = 100
    the intermediate SiLU(g)*u would (|g| ~ 170), at sigma = 1e-3 it would fall into binary16's
    subnormals.  Every token's row is scaled by its own power of two, so all stay within tolerance.
    (The router weights are scaled by 0.02 / sigma, so that logits keep unit scale and a rank gap.)"""
    wl = W.Workload(name="int4-mag-%g-%s" % (sigma, xdt), H=7168, E=64, k=4, I=512, wfmt="int4g32", xdt=xdt,
                    Ts=(48,), seed=919, x_sigma=sigma, wg_sigma=0.02 / sigma)
    T = 48
    say("int4 activation magnitude", wl.name, mode)
    x, _ = oracle.rank_gap_inputs(wl, T)
    layer = build_layer(wl, T)
    out = layer.forward(to_device_act(x, xdt), mode=mode)
    torch.cuda.synchronize()
    ref, ids_ref, _ = oracle_reference(wl, x, np.arange(T))
    assert np.array_equal(layer.topk_ids[:T].cpu().numpy(), ids_ref)
    got = to_f64(out)
    assert np.isfinite(got).all()
    assert_output_close(got, ref, "bf16", wl.name + " " + mode)


# ------------------------------------------------------------------ full-size configurations (sampled tokens)

FULL = [("mixtral", 1, "auto"), ("mixtral", 8, "auto"), ("mixtral", 32, "auto"), ("mixtral", 64, "auto"),
        ("mixtral", 64, "prefill"), ("gptoss", 1, "auto"), ("gptoss", 64, "auto"), ("gptoss", 512, "auto"),
        ("gptoss", 512, "prefill"), ("gptoss", 1024, "auto"),  # 1024: hot experts on the tile kernel
        ("mixtral", 128, "auto"),  # bf16 from 28 rows per expert on average: the tile kernel alone
        # speculative verification blocks of depth + 1 = 2..4 positions (GLM-shaped INT4 layer, resident)
        ("glm", 2, "auto"), ("glm", 3, "decode"), ("glm", 4, "auto"),
        # about 100 experts touched: the shared-activation 4-bit kernel, its INT4 gate/up scales
        # (K = 5120) streamed per stage, its down scales (K = 1536) copied to LDS
        ("glm", 16, "decode")]


@pytest.mark.parametrize("name,T,mode", FULL)
def test_full_size_sampled(name, T, mode):
    wl = W.WORKLOADS[name]
    say("full size", wl.name, "T", T, "mode", mode)
    x, _ = oracle.rank_gap_inputs(wl, T)
    layer = build_layer(wl, T)
    out = layer.forward(to_device_act(x, wl.xdt), mode=mode)
    torch.cuda.synchronize()
    ids_all = layer.topk_ids[:T].cpu().numpy()
    # routing and permutation of every token
    wg, bias = W.router_weights(wl), W.router_bias(wl)
    ids_ref, _ = oracle.topk_gates(oracle.router_logits(wl.xdt, x, wg, bias), wl.k)
    assert np.array_equal(ids_all, ids_ref)
    c, o, p, i = oracle.permute(ids_ref, wl.E)
    assert np.array_equal(layer.offsets.cpu().numpy(), o)
    assert np.array_equal(layer.perm_src[:T * wl.k].cpu().numpy(), p)
    # outputs of up to 64 tokens: every token of a small batch, else rows of every row tile of the
    # hottest experts plus random tokens
    sample = np.arange(T) if T <= 64 else kimi_sample(c, o, p, wl.k, T, n_total=64, seed=T)
    ref, _, _ = oracle_reference(wl, x, sample)
    assert_output_close(to_f64(out)[sample], ref, wl.xdt, "%s T=%d %s" % (wl.name, T, mode))


def kimi_sample(counts, offsets, perm_src, k, T, n_total=256, hottest=3, seed=8192):
    """Tokens to check at full size: for each of the `hottest` experts, the first, middle and last row
    of each of its 192-row tiles (the tile kernel splits an expert's n rows evenly over ceil(n / 192)
    tiles), topped up with seeded random tokens to n_total."""
    pick = set()
    for e in np.argsort(-counts, kind="stable")[:hottest]:
        n = int(counts[e])
        nt = (n + 191) // 192
        for i in range(nt):
            r0, r1 = i * n // nt, (i + 1) * n // nt
            for r in (r0, (r0 + r1) // 2, r1 - 1):
                pick.add(int(perm_src[offsets[e] + r]) // k)
    rng = np.random.default_rng(seed)
    rest = rng.permutation(np.setdiff1d(np.arange(T), sorted(pick)))
    return np.sort(np.concatenate([sorted(pick), rest[:max(0, n_total - len(pick))]]).astype(np.int64))


def test_kimi_prefill_full_size():
    """Kimi-K2-shaped INT4 layer + bf16 shared expert at T=8192: routing and permutation of every
    token bit-exact; the layer output of 256 tokens (every row tile of the three hottest experts
    among them) within tolerance."""
    import concurrent.futures as cf

    wl = W.WORKLOADS["kimi"]
    T = wl.Ts[0]
    say("kimi full size: inputs")
    x, _, lg = oracle.rank_gap_inputs(wl, T, return_logits=True)
    ids_ref, w_ref = oracle.topk_gates(lg, wl.k)
    say("kimi full size: expert weights")
    with cf.ThreadPoolExecutor(max_workers=4) as pool:
        weights = dict(zip(range(wl.E), pool.map(lambda e: W.expert_weights(wl, 0, e), range(wl.E))))
    say("kimi full size: building the device bank")
    layer = build_layer(wl, T, weights=weights)
    say("kimi full size: forward")
    out = layer.forward(to_device_act(x, wl.xdt))
    torch.cuda.synchronize()
    assert np.array_equal(layer.topk_ids.cpu().numpy(), ids_ref)
    np.testing.assert_allclose(layer.topk_w.cpu().numpy(), w_ref, rtol=GATE_RTOL, atol=GATE_ATOL)
    c, o, p, i = oracle.permute(ids_ref, wl.E)
    assert np.array_equal(layer.counts.cpu().numpy(), c)
    assert np.array_equal(layer.perm_src.cpu().numpy(), p)
    assert np.array_equal(layer.inv_perm.cpu().numpy(), i)
    sample = kimi_sample(c, o, p, wl.k, T)
    assert len(sample) >= 256
    say("kimi full size: oracle on", len(sample), "tokens")
    ref, _, _ = oracle_reference(wl, x, sample, weights=weights)
    assert_output_close(to_f64(out)[sample], ref, "bf16", "kimi T=8192")
