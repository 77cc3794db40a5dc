"""The oracle and the C ABI's host code built with AddressSanitizer and
UndefinedBehaviorSanitizer (gcc/g++, CPU only) and run over many shapes.

The host code is linked with stand-ins for the kernel launches
(tests/sanitize/api_stubs.cpp), which also check that every workspace region
lies inside the caller's workspace; no GPU code is built or run here."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _have(tool):
    return shutil.which(tool) is not None


pytestmark = pytest.mark.skipif(not (_have("gcc") and _have("g++")), reason="gcc/g++ not available")


def _run(exe):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    subprocess.run(["gcc", "-std=c11", *SAN, os.path.join(ROOT, "oracle", "art_oracle.c"),
                    os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-o", exe, "-lm", "-lpthread"],
                   check=True)
    _run(exe)


def test_abi_host_code_under_sanitizers(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "kv_cache_bandwidth_amd", "csrc"),
           "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__"]
    objs = []
    for src, cc, std in ((os.path.join(ROOT, "kv_cache_bandwidth_amd", "csrc", "art_api.cpp"), "g++", "-std=c++17"),
                         (os.path.join(ROOT, "tests", "sanitize", "api_stubs.cpp"), "g++", "-std=c++17"),
                         (os.path.join(ROOT, "tests", "sanitize", "api_driver.c"), "gcc", "-std=c11")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        subprocess.run([cc, std, *SAN, *inc, "-c", src, "-o", obj], check=True)
        objs.append(obj)
    exe = str(tmp_path / "api_san")
    subprocess.run(["g++", *SAN, *objs, "-o", exe], check=True)
    _run(exe)
