"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

api.cpp (every host-side argument check) is rebuilt with both sanitizers on
its host pass only and linked with the device objects of the regular build
into a separate shared library; ``host_sanitize_driver.c`` calls every entry
point with arguments that are rejected, or leave nothing to do, before any
launch, and checks the statuses.  No GPU is needed: nothing is launched.
"""

import os
import shutil
import subprocess

import pytest

from linear_attention_state_kda_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def test_abi_host_code_is_sanitizer_clean(tmp_path):
    try:
        hipcc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    objs = [os.path.join(B.BUILD, s + ".o") for s in B.SOURCES if s != "api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("build the library first (linear_attention_state_kda_amd.build)")
    flags = [f for f in B.FLAGS if f != "-O3"] + ["-O1"]
    api_o = str(tmp_path / "api_san.o")
    lib = str(tmp_path / "libkda_san.so")
    drv = str(tmp_path / "driver")

    def run(cmd, **kw):
        r = subprocess.run(cmd, capture_output=True, text=True, **kw)
        assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
        return r

    run([hipcc, "-x", "hip", "-c", os.path.join(B.CSRC, "api.cpp"), "-o", api_o] + flags + SAN)
    run([hipcc, "-shared", "-fPIC", f"--offload-arch={B.ARCH}", "-o", lib, api_o] + objs + SAN)
    run([hipcc, "-x", "c", os.path.join(HERE, "host_sanitize_driver.c"), "-o", drv, "-O1",
         "-I", os.path.join(ROOT, "include"), "-L", str(tmp_path), "-lkda_san",
         f"-Wl,-rpath,{tmp_path}"] + SAN)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([drv], capture_output=True, text=True, env=env, timeout=120)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out
    assert "0 failure(s)" in out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out
