"""Shared helpers for the parity tests: seeded inputs, oracle references, metrics."""
from __future__ import annotations

import sys

import numpy as np

import oracle
from synth import workloads as W


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_l2(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def max_abs_ratio(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-300))


# tolerances on the layer output vs the fp64 oracle
TOL = {
    "bf16": dict(rel_l2=5e-3, max_abs=2e-2),  # bf16 activations
    "f32": dict(rel_l2=1e-5, max_abs=None),   # fp32 activations and fp32 experts
}


def assert_output_close(got, ref, xdt: str, what: str = ""):
    t = TOL[xdt]
    r = rel_l2(got, ref)
    say("  %s rel_l2=%.3e max_abs/max|ref|=%.3e" % (what, r, max_abs_ratio(got, ref)))
    assert r <= t["rel_l2"], "%s: rel-L2 %.3e > %.1e" % (what, r, t["rel_l2"])
    if t["max_abs"] is not None:
        m = max_abs_ratio(got, ref)
        assert m <= t["max_abs"], "%s: max-abs %.3e > %.1e * max|ref|" % (what, m, t["max_abs"])


def to_f64(t) -> np.ndarray:
    """Device/host torch tensor (float32 or bfloat16) -> fp64 numpy."""
    import torch

    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def oracle_reference(wl, x: np.ndarray, sample, layer: int = 0, step: int = 0, weights=None):
    """(out [n, H], ids [n, k], w [n, k]) of the oracle for the sampled tokens, generating only touched experts
    (or taking them from `weights`, a mapping expert -> logical weights)."""
    wg = W.router_weights(wl, layer)
    bias = W.router_bias(wl, layer, step)
    sample = np.asarray(sample, dtype=np.int64)
    xs = np.ascontiguousarray(x[sample])
    lg = oracle.router_logits(wl.xdt, xs, wg, bias)
    ids, _ = oracle.topk_gates(lg, wl.k)
    touched = sorted(set(ids.ravel().tolist()))
    experts = [None] * wl.E
    for e in touched:
        experts[e] = weights[e] if weights is not None else W.expert_weights(wl, layer, e)
    shared = W.shared_weights(wl, layer)
    out, ids2, w = oracle.moe_layer(wl.xdt, x, wg, bias, wl.k, wl.I, experts, shared, wl.I if shared else 0,
                                    sample=sample)
    assert np.array_equal(ids, ids2)
    return out, ids2, w


def small_variant(fmt: str, xdt: str = "bf16", **kw):
    """Reduced layer that still spans several strips, row tiles and a ragged 4-bit chunk tail."""
    base = dict(name="small-%s-%s" % (fmt, xdt), H=224, E=16, k=4, I=352, wfmt=fmt, xdt=xdt, Ts=(40,), seed=777)
    base.update(kw)
    return W.Workload(**base)
