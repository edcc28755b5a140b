"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the host-side C/C++ code: the oracle and
the input generator (gcc), and the expert-cache planner, the lossless encoder and the library's error
state (hipcc, sanitizers on the host code only); each runs a driver that exercises every function and
fails on any report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "mixture_experts_layer_token_amd", "csrc")
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr)
    return r.stdout


def test_oracle_and_generator_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-fopenmp", *SAN, os.path.join(HERE, "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(ROOT, "synth", "synth.c"), "-o", exe, "-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="2")
    assert "ok" in _run([exe], env=env)  # (a nonzero exit code names the failing step of the driver)


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="needs hipcc")
def test_planner_under_sanitizers(tmp_path):
    objs = []
    for src in ("cache.cpp", "errors.cpp", "compress.cpp"):
        o = str(tmp_path / (src + ".o"))
        host_san = [a for f in SAN for a in ("-Xarch_host", f)]
        _run(["hipcc", "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", *host_san, "-c",
              os.path.join(CSRC, src), "-o", o])
        objs.append(o)
    exe = str(tmp_path / "planner_driver")
    _run(["/opt/rocm/llvm/bin/clang++", "-O1", "-g", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__",
          "-I/opt/rocm/include", os.path.join(HERE, "planner_driver.cpp"), *objs, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    # (the HIP runtime's own allocations at exit are not the planner's: leak detection off)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    assert "ok" in _run([exe], env=env)
