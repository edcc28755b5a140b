"""The wait states the prefill tile kernel places around its inline-assembly MFMAs, checked on the
gfx950 assembly hipcc generates for every format and matrix (rules in waitstates.py).  Also checks
that the checker finds a missing wait state in a hand-made sequence."""
import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

import waitstates

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_layer_token_amd", "csrc")
TILE_SOURCES = ["ffn_tile_%s_%s.hip" % (f, m) for f in ("bf16", "mxfp4", "int4g32") for m in ("gu", "down")]


def test_checker_finds_planted_hazards():
    asm = """
kern:
    v_and_or_b32 v4, v1, v2, v3
    v_mfma_f32_16x16x32_f16 a[0:3], v[8:11], v[4:7], a[0:3]
    s_nop 1
    v_accvgpr_read_b32 v9, a2
    s_endpgm
"""
    f = waitstates.functions(asm)["kern"]
    rules = sorted(b[0] for b in waitstates.check(f))
    assert rules == ["R1", "R2"]
    ok = """
kern:
    v_and_or_b32 v4, v1, v2, v3
    s_nop 1
    v_mfma_f32_16x16x32_f16 a[0:3], v[8:11], v[4:7], a[0:3]
    s_nop 7
    s_nop 7
    s_nop 7
    v_accvgpr_read_b32 v9, a2
    s_endpgm
"""
    assert waitstates.check(waitstates.functions(ok)["kern"]) == []
    loop = """
kern:
.LBB0_1:
    v_mfma_f32_16x16x32_f16 a[0:3], v[8:11], v[4:7], a[0:3]
    v_add_u32 v5, v5, v6
    s_cbranch_scc1 .LBB0_1
    s_endpgm
"""
    assert [b[0] for b in waitstates.check(waitstates.functions(loop)["kern"])] == ["R1"]  # around the back-edge


def _asm(src, out_dir):
    out = os.path.join(out_dir, os.path.basename(src) + ".s")
    r = subprocess.run(["hipcc", "-x", "hip", "--offload-arch=gfx950", "--offload-device-only", "-S", "-O3",
                        "-std=c++17", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                        os.path.join(CSRC, src), "-o", out], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="needs hipcc")
def test_tile_kernel_wait_states(tmp_path):
    with cf.ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 1)) as ex:
        files = list(ex.map(lambda s: _asm(s, str(tmp_path)), TILE_SOURCES))
    n_mfma = 0
    for path in files:
        funcs = waitstates.functions(open(path).read())
        kernels = {k: v for k, v in funcs.items() if "ffn_tile_kernel" in k}
        assert kernels, path
        for name, items in kernels.items():
            n_mfma += sum(1 for it in items if not isinstance(it, str) and it.is_mfma)
            bad = waitstates.check(items)
            assert not bad, "%s: %d hazards, first: %s" % (os.path.basename(path), len(bad), bad[:3])
    assert n_mfma > 1000
