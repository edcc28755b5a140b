"""moe_expert_ffn_noalloc (static per-device scratch, no allocation) against moe_expert_ffn with a
caller workspace: the same kernels, so the outputs must be identical bit for bit, on two calls in a
row (the second smaller, in the scratch the first one left behind), in every mode; a call whose
workspace would exceed the static scratch is refused."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402

import mixture_experts_layer_token_amd as moe  # noqa: E402
from mixture_experts_layer_token_amd import api  # noqa: E402
from mixture_experts_layer_token_amd.layer import build_layer, to_device_act  # noqa: E402

from helpers import say, small_variant  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


def _routed(layer, x):
    """topk, offsets and perm_src of x through the layer's router and permutation."""
    T = x.shape[0]
    k = layer.k
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    api.moe_route(x, layer.w_router, layer.bias, k, ids, w)
    counts = torch.empty(layer.E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(layer.E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(T * k, dtype=torch.int32, device="cuda")
    inv = torch.empty(T * k, dtype=torch.int32, device="cuda")
    api.moe_permute(ids, layer.E, counts, offsets, perm, inv)
    return offsets, perm


@pytest.mark.parametrize("fmt", ["bf16", "mxfp4", "int4g32"])
@pytest.mark.parametrize("mode", ["auto", "decode", "prefill"])
def test_noalloc_matches_workspace_call(fmt, mode):
    wl = small_variant(fmt, E=16, k=4)
    layer = build_layer(wl, 130)
    for T in (130, 40):  # the second call is smaller and reuses what the first left in the scratch
        say("noalloc", fmt, mode, "T", T)
        x, _ = oracle.rank_gap_inputs(wl, T, step=T)
        xd = to_device_act(x, wl.xdt)
        offsets, perm = _routed(layer, xd)
        y_ws = torch.full((T * wl.k, wl.H), float("nan"), dtype=torch.float32, device="cuda")
        y_na = torch.full((T * wl.k, wl.H), float("nan"), dtype=torch.float32, device="cuda")
        ws = torch.empty(api.moe_ffn_workspace(layer.desc, T, wl.k, mode), dtype=torch.uint8, device="cuda")
        api.moe_expert_ffn(layer.desc, xd, wl.k, offsets, perm, y_ws, ws, mode=mode)
        api.moe_expert_ffn_noalloc(layer.desc, xd, wl.k, offsets, perm, y_na, mode=mode)
        torch.cuda.synchronize()
        a, b = y_ws.cpu().numpy(), y_na.cpu().numpy()
        assert np.isfinite(a).all()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_noalloc_refuses_more_than_its_scratch():
    wl = small_variant("int4g32", H=4096, I=4096, E=8, k=8)
    d = api.experts_desc(wl.H, wl.I, wl.E, wl.wfmt, None, 1 << 30)
    T = 4096  # h alone: 32768 x 4096 x 2 bytes = 256 MiB
    assert api.moe_ffn_workspace(d, T, wl.k) > (64 << 20)
    with pytest.raises(moe.MoeError) as e:
        api.moe_expert_ffn_noalloc(d, torch.empty((T, wl.H), dtype=torch.bfloat16, device="cuda"), wl.k,
                                   torch.zeros(wl.E + 1, dtype=torch.int32, device="cuda"),
                                   torch.zeros(T * wl.k, dtype=torch.int32, device="cuda"),
                                   torch.empty((1, wl.H), dtype=torch.float32, device="cuda"))
    assert e.value.code == -6 and "static scratch" in str(e.value)
