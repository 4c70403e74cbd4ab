"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the host-side code,
run on the CPU (no GPU needed):

* the fp64 oracle (oracle/gdr_oracle.c) driven over ragged packs, both gate
  forms, grouped heads, with and without h0 / dht (tests/asan/oracle_driver.c);
* libgdr's host code (gdr_api.cpp: planner, workspace sizer, validation of every
  entry point, layout query) with stub kernel launchers that count calls
  (tests/asan/host_driver.cpp).  The planner's tables for 3000 random packs are
  checked against every index the kernels take from them, and no path may reach
  a launch.

Only the host side is instrumented: device code is never built with a sanitizer.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ASAN_DIR = os.path.join(ROOT, "tests", "asan")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang++"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, "%s\n%s%s" % (" ".join(cmd), res.stdout[-3000:], res.stderr[-3000:])
    return res


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    _run(["gcc", "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-g", "-O1", "-fopenmp", "-std=c99",
          "-ffp-contract=off", os.path.join(ROOT, "oracle", "gdr_oracle.c"),
          os.path.join(ASAN_DIR, "oracle_driver.c"), "-o", exe, "-lm"])
    env = dict(ENV, ASAN_OPTIONS="detect_leaks=1", OMP_NUM_THREADS="3")
    out = _run([exe], env=env, timeout=300).stdout
    assert "0 failures" in out


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain not found")
def test_host_code_under_asan(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "chunked_gated_delta_14_amd", "csrc")]
    host_only = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer"]
    objs = []
    for src in (os.path.join(ROOT, "chunked_gated_delta_14_amd", "csrc", "gdr_api.cpp"),
                os.path.join(ASAN_DIR, "host_driver.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC, "--offload-arch=gfx950", "-std=c++17", "-O1", "-g", *host_only, *inc, "-c", src, "-o", obj])
        objs.append(obj)
    exe = str(tmp_path / "host_asan")
    link_sanitizers = "-fsanitize=address,undefined"
    _run([CLANG, link_sanitizers, *objs, "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", exe])
    out = _run([exe], env=ENV, timeout=300).stdout
    assert "0 failures, 0 launches" in out
