"""Compile libmoe.so (HIP, gfx950) in-tree with hipcc.

Every source is compiled as HIP for gfx950 only, with packed-fp32 instruction
generation turned off, then linked into one shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
SO = os.path.join(HERE, "libmoe.so")
BUILD_DIR = os.path.join(HERE, "_build")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH, "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src: str, build_dir: str, extra: tuple) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = ["hipcc", "-x", "hip", *FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr))
    return obj


def build(jobs: int = 8, defines: dict | None = None, out: str | None = None) -> str:
    """Compile and link libmoe.so.  `defines` (name -> value) override the kernels' compile-time
    tile shapes (the MOE_CFG_* macros); `out` puts such a build somewhere else."""
    so = out or SO
    build_dir = BUILD_DIR if out is None else os.path.join(os.path.dirname(os.path.abspath(out)), "_build")
    extra = tuple("-D%s=%s" % kv for kv in sorted((defines or {}).items()))
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, extra), sources()))
    tmp = so + ".tmp%d" % os.getpid()
    r = subprocess.run(["hipcc", "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, so)
    return so


if __name__ == "__main__":
    print(build())
