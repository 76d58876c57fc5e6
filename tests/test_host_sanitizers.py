"""The library's host code (argument validation, capacity, workspace carving, the entry
points' rejection paths) built with AddressSanitizer and UndefinedBehaviorSanitizer and
driven by tests/host_checks.cpp: fuzzed descriptors at and past every limit (including
sizes whose products overflow 64 bits), and every entry point with missing, misaligned or
short arguments.  Host code only: the sanitizer flags reach the host compilation alone
(-Xarch_host before each -fsanitize=), and no GPU call is made."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_mixture_experts_24_amd", "csrc")
SOURCES = ["moe_api.hip", "route.hip", "dispatch.hip", "gemm.hip", "combine.hip",
           "expert_choice.hip"]
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all"]


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


@pytest.mark.timeout(600)
def test_host_code_under_asan_and_ubsan(tmp_path):
    cc = _hipcc()
    if cc is None:
        pytest.skip("hipcc not available")
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-Wno-unused-command-line-argument",
             *HOST_SANITIZE]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([cc, *flags, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    srcs = [os.path.join(CSRC, s) for s in SOURCES] + [os.path.join(ROOT, "tests",
                                                                     "host_checks.cpp")]
    with ThreadPoolExecutor(4) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(tmp_path / "host_checks")
    r = subprocess.run([cc, "--offload-arch=gfx950", *HOST_SANITIZE, *objs, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "0 failures" in r.stdout
