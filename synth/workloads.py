"""Named synthetic workloads: MoE layers shaped like the models the pages discuss.

Shapes (E experts, top-k, shared expert) follow the models named in
"Mixture of experts VRAM: total vs active parameters" (section "How current MoE
models route each token"); the 4-bit expert formats follow the same page
(gpt-oss ships FP4 experts, Kimi INT4 experts).  Values are drawn by
``synth``: activations N(0, 1), expert weights N(0, 0.02) (then block-quantized
for the 4-bit formats), router weights N(0, 0.02); where popularity is skewed, a
per-expert router bias -s * ln(rank) with a seeded rank permutation.

Expert weights are returned in the *logical* layout: gate [I, H], up [I, H],
down [H, I], row-major with the contraction dimension contiguous; the 4-bit
formats as packed nibbles [rows, K/2] (element 2i in the low nibble) plus one
scale per 32 elements along K ([rows, K/32]: E8M0 bytes for MXFP4, bf16 bits for
INT4).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from . import normal, permutation, quant_int4g32, quant_mxfp4, stream_id

WFMTS = ("f32", "bf16", "mxfp4", "int4g32")
XDTS = ("f32", "bf16")


@dataclass(frozen=True)
class Workload:
    name: str
    H: int
    E: int
    k: int
    I: int
    wfmt: str
    xdt: str
    Ts: tuple
    seed: int
    x_sigma: float = 1.0
    w_sigma: float = 0.02
    wg_sigma: float = 0.02
    zipf_s: float | None = None  # per-expert bias -s*ln(rank); None = no bias
    shared: bool = False  # one always-on bf16 shared expert with inter I
    layers: int = 1
    steps: int = 1
    rerank_every: int = 0  # offload workload: ranks redrawn every this many steps
    cache_frac: float = 0.0  # offload workload: HBM cache size as a fraction of the bank

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    # tiny fp32 layer: exhaustively checkable on the CPU
    "tiny": Workload("tiny-fp32", H=256, E=8, k=2, I=512, wfmt="f32", xdt="f32", Ts=(16,), seed=101),
    # Mixtral-8x7B-shaped, bf16 experts, uniform-random router, decode batches
    "mixtral": Workload("mixtral-8x7b-bf16", H=4096, E=8, k=2, I=14336, wfmt="bf16", xdt="bf16",
                        Ts=(1, 8, 32, 64), seed=202),
    # gpt-oss-120b-shaped, MXFP4 experts, Zipf(1.1) expert popularity
    "gptoss": Workload("gpt-oss-120b-mxfp4", H=2880, E=128, k=4, I=2880, wfmt="mxfp4", xdt="bf16",
                       Ts=(1, 64, 512), seed=303, zipf_s=1.1),
    # Kimi-K2-shaped, INT4 group-32 experts + one bf16 shared expert, prefill
    "kimi": Workload("kimi-k2-int4-prefill", H=7168, E=384, k=8, I=2048, wfmt="int4g32", xdt="bf16",
                     Ts=(8192,), seed=404, shared=True),
    # GLM-shaped offloaded bank: 8 layers, INT4 group-32, Zipf(1.2) drifting every 64 steps
    "glm": Workload("glm-offload-int4", H=5120, E=256, k=8, I=1536, wfmt="int4g32", xdt="bf16",
                    Ts=(1, 16), seed=505, zipf_s=1.2, layers=8, steps=256, rerank_every=64,
                    cache_frac=0.25),
}


def act_dtype(wl: Workload) -> str:
    return wl.xdt


def router_weights(wl: Workload, layer: int = 0) -> np.ndarray:
    """Wg [E, H] in the activation dtype (float32, or bf16 bits as uint16)."""
    return normal(wl.seed, stream_id(wl.name, "wg", layer), (wl.E, wl.H), wl.wg_sigma, wl.xdt)


def router_bias(wl: Workload, layer: int = 0, step: int = 0):
    """Per-expert router bias b_e = -s * ln(rank_e), rank = seeded permutation + 1; None without skew."""
    if wl.zipf_s is None:
        return None
    epoch = step // wl.rerank_every if wl.rerank_every else 0
    rank = permutation(wl.seed, stream_id(wl.name, "rank", layer, epoch), wl.E) + 1
    return np.array([-wl.zipf_s * math.log(r) for r in rank], dtype=np.float32)


def activation_rows(wl: Workload, layer: int, step: int, rows, attempts=None) -> np.ndarray:
    """Rows of x; row t is drawn from its own stream (t, attempt) so single rows can be redrawn."""
    rows = list(rows)
    dt = np.float32 if wl.xdt == "f32" else np.uint16
    out = np.empty((len(rows), wl.H), dtype=dt)
    for i, t in enumerate(rows):
        a = 0 if attempts is None else int(attempts[i])
        out[i] = normal(wl.seed, stream_id(wl.name, "x", layer, step, t, a), (wl.H,), wl.x_sigma, wl.xdt)
    return out


def activations(wl: Workload, T: int, layer: int = 0, step: int = 0, attempts=None) -> np.ndarray:
    """x [T, H] in the activation dtype."""
    return activation_rows(wl, layer, step, range(T), attempts)


def _matrix(wl: Workload, fmt: str, stream: int, rows: int, K: int):
    if fmt == "f32":
        return normal(wl.seed, stream, (rows, K), wl.w_sigma, "f32"), None
    if fmt == "bf16":
        return normal(wl.seed, stream, (rows, K), wl.w_sigma, "bf16"), None
    if fmt == "mxfp4":
        return quant_mxfp4(wl.seed, stream, rows, K, wl.w_sigma)
    if fmt == "int4g32":
        return quant_int4g32(wl.seed, stream, rows, K, wl.w_sigma)
    raise ValueError(fmt)


def expert_weights(wl: Workload, layer: int, e: int) -> dict:
    """Logical weights of routed expert e: {'fmt', 'w': [gate, up, down], 's': [scales or None]*3}."""
    shapes = ((wl.I, wl.H), (wl.I, wl.H), (wl.H, wl.I))
    w, s = [], []
    for m, (rows, K) in enumerate(shapes):
        a, b = _matrix(wl, wl.wfmt, stream_id(wl.name, "w", layer, e, m), rows, K)
        w.append(a)
        s.append(b)
    return {"fmt": wl.wfmt, "w": w, "s": s}


def shared_weights(wl: Workload, layer: int = 0) -> dict | None:
    """The always-on shared expert (bf16, inter I), or None."""
    if not wl.shared:
        return None
    shapes = ((wl.I, wl.H), (wl.I, wl.H), (wl.H, wl.I))
    w = [normal(wl.seed, stream_id(wl.name, "shared", layer, m), shp, wl.w_sigma, "bf16")
         for m, shp in enumerate(shapes)]
    return {"fmt": "bf16", "w": w, "s": [None, None, None]}


def package_bytes(wl: Workload, fmt: str | None = None) -> int:
    """Bytes of one expert's weights including block scales (6HI for bf16, 4.25 / 4.5 bit per weight for 4-bit)."""
    fmt = fmt or wl.wfmt
    n = 3 * wl.H * wl.I
    return {"f32": 4 * n, "bf16": 2 * n, "mxfp4": n // 2 + n // 32, "int4g32": n // 2 + 2 * (n // 32)}[fmt]
