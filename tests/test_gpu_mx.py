"""GPU parity of the block-scaled MXFP4 mode (MOE_FFN_DECODE_MX): FP4 weights straight into
v_mfma_scale_f32_16x16x128_f8f6f4, activations and h as two MXFP8 terms per 32-element block.

Tolerance of this mode: each activation element is held to within 2^-8 of its magnitude (the second
E4M3 term holds the first one's remainder, at most 2^-4 of the element, to 2^-4 of itself), where bf16
holds it to 2^-9, and this rounding applies to both x and h; the bar is therefore twice the bf16 one:
rel-L2 <= 1e-2 and max-abs <= 4e-2 * max|ref| against the fp64 oracle.  Routing is the router's
(bit-exact as in every mode).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from synth import workloads as W  # noqa: E402

import mixture_experts_layer_token_amd as moe  # noqa: E402
from mixture_experts_layer_token_amd.layer import build_layer, to_device_act  # noqa: E402

from helpers import max_abs_ratio, oracle_reference, rel_l2, say, small_variant, to_f64  # noqa: E402

MX_REL_L2, MX_MAX_ABS = 1e-2, 4e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


def check(got, ref, what):
    r, m = rel_l2(got, ref), max_abs_ratio(got, ref)
    say("  %s rel_l2=%.3e max_abs/max|ref|=%.3e" % (what, r, m))
    assert r <= MX_REL_L2 and m <= MX_MAX_ABS, what


@pytest.mark.parametrize("T", [1, 3, 40, 130])
@pytest.mark.parametrize("xdt", ["bf16", "f32"])
def test_mx_layer_small(T, xdt):
    """Ragged K in both matrices (H = 224, I = 352: 7 and 11 blocks of 32, partial 128-wide chunks),
    one and two M tiles."""
    wl = small_variant("mxfp4", xdt)
    say("mx layer small", wl.name, "T", T)
    x, _ = oracle.rank_gap_inputs(wl, T)
    layer = build_layer(wl, T)
    out = layer.forward(to_device_act(x, xdt), mode="decode_mx")
    torch.cuda.synchronize()
    ref, ids_ref, _ = oracle_reference(wl, x, np.arange(T))
    assert np.array_equal(layer.topk_ids[:T].cpu().numpy(), ids_ref)
    check(to_f64(out), ref, "%s T=%d" % (wl.name, T))


def test_mx_many_experts_and_large_values():
    """E = 128, top-8 (most experts touched), activations of std 100 (the per-block scales carry them)."""
    wl = small_variant("mxfp4", E=128, k=8, name="mx-wide", x_sigma=100.0, wg_sigma=2e-4)
    T = 200
    say("mx many experts")
    x, _ = oracle.rank_gap_inputs(wl, T)
    layer = build_layer(wl, T)
    out = layer.forward(to_device_act(x, "bf16"), mode="decode_mx")
    torch.cuda.synchronize()
    ref, ids_ref, _ = oracle_reference(wl, x, np.arange(T))
    assert np.array_equal(layer.topk_ids[:T].cpu().numpy(), ids_ref)
    check(to_f64(out), ref, wl.name)


@pytest.mark.parametrize("T", [1, 64])
def test_mx_gptoss_full_size(T):
    """gpt-oss-shaped layer (hidden 2880 = 22.5 chunks of 128, 128 experts, top-4) at full size."""
    wl = W.WORKLOADS["gptoss"]
    say("mx gpt-oss full size T", T)
    x, _ = oracle.rank_gap_inputs(wl, T)
    layer = build_layer(wl, T)
    out = layer.forward(to_device_act(x, wl.xdt), mode="decode_mx")
    torch.cuda.synchronize()
    sample = np.arange(T) if T <= 16 else np.arange(0, T, 4)
    ref, ids_ref, _ = oracle_reference(wl, x, sample)
    assert np.array_equal(layer.topk_ids[:T].cpu().numpy()[sample], ids_ref)
    check(to_f64(out)[sample], ref, "gpt-oss T=%d" % T)


def test_mx_mode_refuses_other_formats():
    wl = small_variant("int4g32")
    layer = build_layer(wl, 4)
    x, _ = oracle.rank_gap_inputs(wl, 4)
    with pytest.raises(moe.MoeError) as e:
        layer.forward(to_device_act(x, "bf16"), mode="decode_mx")
    assert e.value.code == -2
