"""GPU parity of moe_expert_ffn alone, on hand-built groupings that give the experts every row count
the kernels treat differently, against oracle.ffn expert by expert.

The prefill (MFMA tile) kernel cuts an expert with n rows into ceil(n / 192) row tiles that split the
rows evenly and runs the variant with ceil(rows / 16) 16-row MFMA tiles, so:
  - counts 1..192 reach every variant (1..12 MFMA row tiles) with every ragged tail (rows mod 16);
  - counts 193..384 are experts split in two tiles (of 97..192 rows);
  - counts above 384 split in three or more.
The streaming (decode) kernel cuts the same experts into 16- or 32-row tiles.  Rows are gathered
through a shuffled perm_src (k = 2), H = 224 and I = 352 leave a ragged 4-bit package chunk in both
contractions and a ragged column tile in both matrices.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from synth import workloads as W  # noqa: E402

import mixture_experts_layer_token_amd as moe  # noqa: E402
from mixture_experts_layer_token_amd import api  # noqa: E402
from mixture_experts_layer_token_amd.layer import pack_bank, to_device_act  # noqa: E402

from helpers import assert_output_close, say, small_variant  # noqa: E402

SPLIT_COUNTS = [193, 200, 250, 300, 383, 384, 385, 500, 1000]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


def grouping(counts, k, seed):
    """offsets [E+1] and a shuffled perm_src over T*k flat indices for the given per-expert counts."""
    n = int(np.sum(counts))
    assert n % k == 0
    rng = np.random.default_rng(seed)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    perm_src = rng.permutation(n).astype(np.int32)
    return offsets, perm_src, n // k


def run_rows(fmt, mode, counts, k=2, seed=5):
    wl = small_variant(fmt, E=len(counts), name="rows-%s" % fmt)
    offsets, perm_src, T = grouping(counts, k, seed)
    say("ffn rows", fmt, mode, "E", wl.E, "T", T, "pairs", T * k)
    bank = pack_bank(wl, 0, list(range(wl.E)))
    stride = bank.shape[1]
    packages = torch.from_numpy(bank).cuda()
    desc = api.experts_desc(wl.H, wl.I, wl.E, fmt, packages, stride)
    x_host = W.activations(wl, T)
    x = to_device_act(x_host, wl.xdt)
    d_off = torch.from_numpy(offsets).cuda()
    d_perm = torch.from_numpy(perm_src).cuda()
    y = torch.full((T * k, wl.H), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(api.moe_ffn_workspace(desc, T, k, mode), dtype=torch.uint8, device="cuda")
    api.moe_expert_ffn(desc, x, k, d_off, d_perm, y, ws, mode=mode)
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    xd = oracle.decode_act(wl.xdt, x_host)
    for e in range(wl.E):
        if counts[e] == 0:
            continue
        rows = perm_src[offsets[e]:offsets[e + 1]] // k
        ref = oracle.ffn(W.expert_weights(wl, 0, e), wl.H, wl.I, xd[rows])
        blk = got[offsets[e]:offsets[e + 1]]
        assert np.isfinite(blk).all(), "expert %d (%d rows): rows left unwritten" % (e, counts[e])
        if counts[e] in (1, 16, 17, 192) or counts[e] > 192:
            assert_output_close(blk, ref, "bf16", "%s %s expert %d rows %d" % (fmt, mode, e, counts[e]))
        else:
            _quiet_close(blk, ref, fmt, mode, e, counts[e])


def _quiet_close(got, ref, fmt, mode, e, c):
    """The output tolerance (bf16 activations) without a line per expert."""
    d = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    m = np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-300)
    assert d <= 5e-3 and m <= 2e-2, "%s %s expert %d rows %d: rel-L2 %.3e max-abs %.3e" % (fmt, mode, e, c, d, m)


@pytest.mark.parametrize("fmt", ["bf16", "mxfp4", "int4g32"])
@pytest.mark.parametrize("mode", ["prefill", "decode"])
def test_ffn_every_row_count(fmt, mode):
    rng = np.random.default_rng(17)
    counts = list(range(1, 193)) + SPLIT_COUNTS
    if sum(counts) % 2:
        counts.append(1)
    counts = rng.permutation(np.array(counts, dtype=np.int64))  # hot and cold experts interleaved
    run_rows(fmt, mode, counts)


@pytest.mark.parametrize("fmt", ["bf16", "mxfp4", "int4g32"])
def test_ffn_empty_experts_between(fmt):
    """Experts with no rows between busy ones (and at both ends), in the auto mode's hybrid regime:
    a few experts above the streaming split go to the tile kernel, the rest stream."""
    counts = np.array([0, 3, 0, 0, 200, 1, 0, 64, 65, 0, 130, 7, 0, 0, 400, 0], dtype=np.int64)
    if counts.sum() % 2:
        counts[1] += 1
    if fmt == "bf16":
        # bf16 experts all go to the tile kernel from 28 rows per expert on average: more empty experts
        counts = np.concatenate([counts, np.zeros(24, np.int64)])
    run_rows(fmt, "auto", counts, seed=9)
