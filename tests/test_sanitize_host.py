"""The host-side argument checks of the C ABI built with AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only): api.hip compiled for the host alone,
the launchers replaced by counting stand-ins (tests/sanitize/stubs.cpp), driven
by tests/sanitize/validate.cpp through every rejection path and a few accepted
calls.  Any out-of-bounds access, overflow or other undefined behaviour in the
checks aborts the driver."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    pytest.skip("hipcc not available")


def test_argument_checks_under_asan_and_ubsan(tmp_path):
    inc = [f"-I{ROOT}/include", f"-I{ROOT}/rank_kv_cache_lrkv_amd/csrc"]
    api_o = str(tmp_path / "api.o")
    # host-only compilation: each sanitizer flag applies to the host pass alone
    host_san = [x for f in SAN for x in ("-Xarch_host", f)]
    subprocess.run([_hipcc(), "--cuda-host-only", "-O1", "-g", "-std=c++17", "-fPIC", *host_san, *inc, "-c",
                    f"{ROOT}/rank_kv_cache_lrkv_amd/csrc/api.hip", "-o", api_o], check=True,
                   capture_output=True, text=True)
    stubs_o = str(tmp_path / "stubs.o")
    subprocess.run([_hipcc(), "--cuda-host-only", "-x", "hip", "-O1", "-g", "-std=c++17", "-fPIC", *host_san, *inc,
                    "-c", f"{HERE}/stubs.cpp", "-o", stubs_o], check=True, capture_output=True, text=True)
    exe = str(tmp_path / "validate")
    subprocess.run(["g++", "-O1", "-g", "-std=c++17", *SAN, f"-I{ROOT}/include", f"{HERE}/validate.cpp", stubs_o,
                    api_o, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe], check=True,
                   capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stderr[-3000:]
    assert "checks passed" in r.stdout
