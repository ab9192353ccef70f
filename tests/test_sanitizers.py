"""AddressSanitizer and UndefinedBehaviorSanitizer runs on the CPU (no GPU).

  * The oracle (oracle/moe_oracle.c) built with -fsanitize=address,undefined
    and run through every function by tests/sanitize/oracle_selftest.c.
  * The C ABI's host code (sparse_moe_amd/csrc/capi.hip) built with both
    sanitizers for its host side only, linked with the library's other
    objects, and run through the argument validation of every entry point by
    tests/sanitize/capi_selftest.cpp (every call is rejected before anything
    is enqueued, so no device is needed).
Any memory error, leak or undefined operation makes the program exit non-zero."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-3000:], r.stderr[-3000:])
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_selftest")
    _run(["gcc", "-std=c11", "-D_DEFAULT_SOURCE", "-O1", "-g", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-Wall", "-Wextra",
          "-Werror", "-I", os.path.join(ROOT, "oracle"), os.path.join(HERE, "oracle_selftest.c"),
          os.path.join(ROOT, "oracle", "moe_oracle.c"), "-lm", "-o", exe])
    r = _run([exe], env=ENV)
    assert "passed" in r.stdout


def test_c_abi_validation_under_asan_ubsan(tmp_path):
    objs = os.path.join(ROOT, "sparse_moe_amd", "_build")
    others = sorted(os.path.join(objs, f) for f in os.listdir(objs)
                    if f.endswith(".hip.o") and f != "capi.hip.o") if os.path.isdir(objs) else []
    if not os.path.exists(HIPCC) or not others:
        pytest.skip("hipcc or the library's objects (python -m sparse_moe_amd.build) missing")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "sparse_moe_amd", "csrc")]
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    capi = str(tmp_path / "capi.o")
    drv = str(tmp_path / "drv.o")
    exe = str(tmp_path / "capi_selftest")
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *san, "-Xclang",
          "-target-feature", "-Xclang", "-packed-fp32-ops", *inc, "-c",
          os.path.join(ROOT, "sparse_moe_amd", "csrc", "capi.hip"), "-o", capi])
    _run([HIPCC, "-O1", "-g", "-std=c++17", *san, *inc, "-x", "c++", "-c",
          os.path.join(HERE, "capi_selftest.cpp"), "-o", drv])
    _run([HIPCC, "--offload-arch=gfx950", *san, capi, drv, *others, "-o", exe])
    r = _run([exe], env=ENV)
    assert "passed" in r.stdout
