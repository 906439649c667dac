"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The library is rebuilt with the sanitizers on its host code only (`-Xarch_host` before
each `-fsanitize`; device code is untouched and never launched), and the instrumented
driver tests/host_checks.cpp calls every host path of the C ABI: argument checks,
launch-plan and workspace arithmetic over a sweep of sizes (prefixes up to 2^30 keys,
batches up to 1024), the cost-table lookup and the budget bars.  A sanitizer report or
a wrong status fails the test.  The build is cached per source hash in the system's
temporary directory."""

import glob
import hashlib
import os
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang++"


def _sources():
    return sorted(glob.glob(os.path.join(ROOT, "tree_attention_verify_ancestor_amd", "csrc", "*"))) + \
        [os.path.join(ROOT, "include", "treeverify.h"), os.path.join(ROOT, "tests", "host_checks.cpp")]


def _build_dir():
    h = hashlib.sha256()
    for p in _sources():
        h.update(open(p, "rb").read())
    d = os.path.join(tempfile.gettempdir(), "treeverify_sanitized_" + h.hexdigest()[:16])
    os.makedirs(d, exist_ok=True)
    return d


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain missing")
def test_host_code_under_asan_and_ubsan():
    d = _build_dir()
    lib = os.path.join(d, "libtreeverify_sanitized.so")
    exe = os.path.join(d, "host_checks")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined"]
    if not os.path.exists(lib):
        srcs = sorted(glob.glob(os.path.join(ROOT, "tree_attention_verify_ancestor_amd", "csrc", "*.hip")))
        cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-shared", "-std=c++17",
               "-Wno-inline-asm", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *san,
               "-I", os.path.join(ROOT, "include"), *srcs, "-o", lib + ".tmp"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        os.replace(lib + ".tmp", lib)
    if not os.path.exists(exe):
        cmd = [CLANG, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
               "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__",
               "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
               os.path.join(ROOT, "tests", "host_checks.cpp"), lib, "-Wl,-rpath," + d, "-o", exe + ".tmp"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        os.replace(exe + ".tmp", exe)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0 and "host checks ok" in r.stdout, (r.stdout[-2000:] + r.stderr[-4000:])
