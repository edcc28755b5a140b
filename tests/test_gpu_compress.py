"""GPU parity of the lossless package decoder (moe_decompress_packages): every decoded package
equals the original bytes exactly.  Blobs are the oracle encoder's (the library's host encoder
matches it byte for byte in test_abi_cpu.py); the expected output is the input package itself."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from synth import workloads as W  # noqa: E402

import mixture_experts_layer_token_amd as moe  # noqa: E402

from helpers import say  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


def _bf16(a):
    return (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _raw(kind, n_vals, seed):
    rng = np.random.default_rng(seed)
    if kind == "gaussian":
        v = _bf16(rng.normal(0, 0.02, n_vals))
    elif kind == "bits":
        v = rng.integers(0, 1 << 16, n_vals, dtype=np.uint16)
    elif kind == "specials":
        v = rng.choice(np.array([0, 0x8000, 0x7F80, 0xFF80, 0x7FC1, 0x0001, 0x8080, 0x3F80, 0x0680], np.uint16),
                       n_vals)
    else:  # gaussian with scattered escapes: zeros, subnormals, tiny values, and chunks at the raw boundary
        v = _bf16(rng.normal(0, 0.02, n_vals))
        idx = rng.integers(0, n_vals, n_vals // 300)
        v[idx] = rng.choice(np.array([0, 0x8000, 0x0003, 0x0080, 0x2000], np.uint16), idx.size)
        for c, n_esc in enumerate((0, 1, 15, 16, 17, 63, 64, 65, 240, 241, 511)):
            if (c + 1) * 512 <= n_vals:
                ch = v[c * 512:(c + 1) * 512]
                ch[:] = 0x5F00
                ch[0] = 0x6400
                ch[1:1 + n_esc] = 0x0080
    return v.view(np.uint8)


def _run(raws, pairs_host, n_dst, stride_dst):
    blobs = [oracle.xw4_encode(r) for r in raws]
    stride = (max(b.size for b in blobs) + 255) // 256 * 256
    src = np.zeros((len(blobs), stride), np.uint8)
    for i, b in enumerate(blobs):
        src[i, :b.size] = b
    d_src = torch.from_numpy(src).cuda()
    d_dst = torch.full((n_dst, stride_dst), 0xAB, dtype=torch.uint8, device="cuda")
    pairs = torch.tensor(pairs_host, dtype=torch.int32, device="cuda").reshape(-1, 2)
    moe.moe_decompress_packages(d_src, stride, d_dst, stride_dst, pairs, raws[0].size)
    torch.cuda.synchronize()
    return d_dst.cpu().numpy(), [b.size / r.size for b, r in zip(blobs, raws)]


@pytest.mark.parametrize("kind", ["gaussian", "bits", "specials", "escapes"])
def test_decompress_bit_exact(kind):
    n_vals = 512 * 1200  # 1200 chunks: a ragged last workgroup (16 chunks per workgroup)
    raws = [_raw(kind, n_vals, seed) for seed in range(4)]
    raw_bytes = raws[0].size
    stride_dst = raw_bytes + 4096
    # sources 0..3 to destinations 2, 0, (skipped), 3; a pair with a negative destination is skipped too
    pairs = [0, 2, 1, 0, -1, 1, 3, 3, 2, -5]
    got, ratios = _run(raws, pairs, 5, stride_dst)
    say("decompress", kind, "ratios", ["%.4f" % r for r in ratios])
    for src_i, dst_i in ((0, 2), (1, 0), (3, 3)):
        assert np.array_equal(got[dst_i, :raw_bytes], raws[src_i]), (src_i, dst_i)
        assert (got[dst_i, raw_bytes:] == 0xAB).all()
    assert (got[1] == 0xAB).all() and (got[4] == 0xAB).all()


def test_decompress_full_size_glm_bf16_experts():
    """Three GLM-shaped experts (H 5120, I 1536) in bf16: 47 MB each."""
    wl = W.WORKLOADS["glm"].with_(wfmt="bf16", name="glm-bf16")
    raws = []
    for e in range(3):
        ex = W.expert_weights(wl, 0, e)
        raws.append(np.concatenate([np.ascontiguousarray(a).view(np.uint8).ravel() for a in ex["w"]]))
    assert raws[0].size == 6 * wl.H * wl.I
    got, ratios = _run(raws, [0, 1, 1, 2, 2, 0], 3, raws[0].size)
    say("decompress glm bf16 ratios", ["%.4f" % r for r in ratios])
    assert all(0.75 <= r < 0.76 for r in ratios)
    for src_i, dst_i in ((0, 1), (1, 2), (2, 0)):
        assert np.array_equal(got[dst_i], raws[src_i])


def test_decompress_nothing_to_do():
    d = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    pairs = torch.zeros((0, 2), dtype=torch.int32, device="cuda")
    moe.moe_decompress_packages(d, 1024, d, 1024, pairs, 1024)
    torch.cuda.synchronize()
    assert int(d.sum()) == 0
