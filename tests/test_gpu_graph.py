"""A layer forward captured in a HIP graph and replayed gives the eager result, replay after
replay, with other eager work and synchronisations between the replays."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from synth import workloads as W  # noqa: E402

import mixture_experts_layer_token_amd as moe  # noqa: E402
from mixture_experts_layer_token_amd.layer import build_layer, to_device_act  # noqa: E402

from helpers import say, small_variant  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


# (T = 200 with 4-bit experts: the AUTO hybrid, whose tile share runs on the library's helper
# stream, forked and joined inside the capture)
@pytest.mark.parametrize("fmt,T", [("bf16", 8), ("mxfp4", 40), ("int4g32", 300), ("bf16", 1), ("int4g32", 200),
                                   ("mxfp4", 200)])
def test_graph_replay_matches_eager(fmt, T):
    wl = small_variant(fmt)
    say("graph replay", fmt, "T", T)
    layer = build_layer(wl, T)
    x = to_device_act(W.activations(wl, T, 0, 11), wl.xdt)
    x_other = to_device_act(W.activations(wl, T, 0, 12), wl.xdt)
    ref = layer.forward(x).clone()
    other_ref = layer.forward(x_other).clone()
    torch.cuda.synchronize()

    out = torch.empty_like(x)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.forward(x, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(x, out)
    for rep in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "replay %d" % rep
        # eager work on the same buffers between replays
        o2 = layer.forward(x_other)
        torch.cuda.synchronize()
        assert torch.equal(o2, other_ref)
    del g
    assert np.isfinite(ref.float().cpu().numpy()).all()
