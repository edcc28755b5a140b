"""The seeded generator: determinism, random access, distributions, quantizers."""
import hashlib
import math

import numpy as np

import synth
from synth import workloads as W


def test_splitmix64_reference_sequence():
    # SplitMix64 with state 0: the first outputs of the published generator
    want = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    assert [synth.lib().synth_draw_key(0, i) for i in range(3)] == want


def test_determinism_and_random_access():
    a = synth.normal(7, 99, (1000,), 1.0, "f64")
    b = synth.normal(7, 99, (1000,), 1.0, "f64")
    assert np.array_equal(a, b)
    c = synth.normal(7, 99, (300,), 1.0, "f64", offset=401)
    assert np.array_equal(c, a[401:701])
    d = synth.normal(8, 99, (1000,), 1.0, "f64")
    assert not np.array_equal(a, d)


def test_normal_moments():
    z = synth.normal(1, 2, (400000,), 1.0, "f64")
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01
    assert abs(np.mean(np.abs(z) > 1.96) - 0.05) < 0.003


def test_bf16_and_f32_rounding():
    d = synth.normal(3, 4, (20000,), 1.0, "f64")
    f = synth.normal(3, 4, (20000,), 1.0, "f32")
    assert np.array_equal(f, d.astype(np.float32))
    h = synth.normal(3, 4, (20000,), 1.0, "bf16")
    # value of the bf16 pattern is the nearest bf16 to the double (ties to even)
    v = (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ulp = np.array([math.ldexp(1.0, math.frexp(abs(x))[1] - 8) for x in d])
    err = np.abs(v - d)
    assert np.all(err <= ulp / 2)


def test_mxfp4_quantizer_properties():
    codes, scales = synth.quant_mxfp4(5, 6, 64, 256, 0.02)
    w = synth.normal(5, 6, (64, 256), 0.02, "f64")
    amax = np.abs(w.reshape(64, 8, 32)).max(axis=2)
    X = scales.astype(np.int64) - 127
    assert np.array_equal(X, np.floor(np.log2(amax)).astype(np.int64) - 2)
    # decoded value within half an E2M1 step of the original (saturation only above 6 * 2^X)
    table = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])
    lo, hi = codes & 15, codes >> 4
    el = np.empty((64, 256), dtype=np.int64)
    el[:, 0::2], el[:, 1::2] = lo, hi
    dec = table[el] * np.exp2(np.repeat(X, 32, axis=1))
    step = np.exp2(np.repeat(X, 32, axis=1))  # largest E2M1 gap is 2 units: error <= 1 unit
    assert np.all((np.abs(dec - w) <= step + 1e-18) | (np.abs(w) > 6 * step))


def test_int4_quantizer_properties():
    codes, scales = synth.quant_int4g32(5, 7, 32, 128, 0.02)
    w = synth.normal(5, 7, (32, 128), 0.02, "f64")
    amax = np.abs(w.reshape(32, 4, 32)).max(axis=2)
    s = (scales.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.all(np.abs(s - amax / 7) <= np.abs(amax / 7) * 2.0 ** -8)
    el = np.empty((32, 128), dtype=np.int64)
    el[:, 0::2], el[:, 1::2] = codes & 15, codes >> 4
    q = np.where(el >= 8, el - 16, el)
    assert q.min() >= -7 and q.max() <= 7
    S = np.repeat(s, 32, axis=1)
    assert np.all(np.abs(q * S - w) <= S / 2 + 1e-12 * S + np.maximum(0, np.abs(w) - 7 * S))


def test_workload_streams_hash_stable():
    wl = W.WORKLOADS["tiny"]
    h = hashlib.sha256()
    h.update(W.activations(wl, 16).tobytes())
    h.update(W.router_weights(wl).tobytes())
    h.update(W.expert_weights(wl, 0, 3)["w"][2].tobytes())
    h2 = hashlib.sha256()
    h2.update(W.activations(wl, 16).tobytes())
    h2.update(W.router_weights(wl).tobytes())
    h2.update(W.expert_weights(wl, 0, 3)["w"][2].tobytes())
    assert h.hexdigest() == h2.hexdigest()


def test_zipf_bias_and_permutation():
    wl = W.WORKLOADS["gptoss"]
    b = W.router_bias(wl)
    ranks = np.rint(np.exp(-b / wl.zipf_s)).astype(int)
    assert sorted(ranks.tolist()) == list(range(1, wl.E + 1))
    glm = W.WORKLOADS["glm"]
    assert np.array_equal(W.router_bias(glm, 0, 0), W.router_bias(glm, 0, 63))
    assert not np.array_equal(W.router_bias(glm, 0, 63), W.router_bias(glm, 0, 64))


def test_package_bytes_formula():
    assert W.package_bytes(W.WORKLOADS["mixtral"]) == 352321536
    assert W.package_bytes(W.WORKLOADS["gptoss"]) == 13219200
    assert W.package_bytes(W.WORKLOADS["kimi"]) == 24772608
    assert W.package_bytes(W.WORKLOADS["glm"]) == 13271040
    assert W.package_bytes(W.WORKLOADS["tiny"]) == 1572864
