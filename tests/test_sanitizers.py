"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only):

* the fp64 oracle (oracle/laoracle.c) driven through every routine by
  tests/sanitize/oracle_main.c, built with gcc;
* the C ABI's host side (la_api.cpp: argument checks, planning, workspace
  sizing, dispatch) driven through every entry point by
  tests/sanitize/api_main.cpp, with the kernel launchers replaced by stubs
  that check their arguments; built with hipcc, the sanitizers on the host
  pass only (the device pass is not instrumented).

Each build runs in a fresh process; a sanitizer report makes it exit non-zero.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(cmd, env=None, timeout=300):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-4000:], r.stderr[-4000:])
    return r.stdout


def _env():
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    env["OMP_NUM_THREADS"] = "2"
    return env


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    _run(["gcc", "-O1", "-g", "-std=c99", "-fopenmp", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          os.path.join(SAN, "oracle_main.c"), os.path.join(ROOT, "oracle", "laoracle.c"), "-lm", "-o", exe])
    out = _run([exe], env=_env())
    assert "OK (0 failures)" in out, out


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_c_abi_host_path_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "api_asan")
    csrc = os.path.join(ROOT, "kernelized_linear_attention_chunked_amd", "csrc")
    _run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-sanitize-recover=all",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
          "-I", os.path.join(ROOT, "include"), "-I", csrc,
          os.path.join(SAN, "api_main.cpp"), os.path.join(csrc, "la_api.cpp"), "-o", exe])
    out = _run([exe], env=_env())
    assert out.strip().startswith("OK:"), out
