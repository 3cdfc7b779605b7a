"""The host layer under AddressSanitizer and UndefinedBehaviorSanitizer.

oxa_host.cpp (argument checks, workspace layouts, launch set-up) is built with
both sanitizers on its host pass (paged_attention_02_amd.build.
build_host_sanitized) and the host-validation and binding-shape suites run
against that build in a child process with the ASan runtime preloaded: any
out-of-bounds access, use after free or undefined behaviour in the checks
aborts the child.  CPU only: on a GPU host the validation suite itself does not
run (its pointers are fake).
"""
import glob
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(torch.cuda.is_available(),
                                reason="host-layer sanitizer run is for GPU-less hosts")


def asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


CHILD = r"""
import sys
import paged_attention_02_amd as oxa
oxa.lib()
maps = open("/proc/self/maps").read()
assert "liboxa_host_sanitized.so" in maps, "the sanitized build is not the one loaded"
assert "libclang_rt.asan" in maps, "the ASan runtime is not loaded"
import pytest
sys.exit(pytest.main(["tests/test_host_validation.py", "tests/test_binding_shapes.py", "-q",
                      "-x", "-p", "no:cacheprovider"]))
"""


def test_host_layer_is_clean_under_asan_and_ubsan():
    rt = asan_runtime()
    if rt is None:
        pytest.skip("no ASan runtime in this ROCm installation")
    from paged_attention_02_amd import build
    lib = build.build_host_sanitized()
    env = dict(os.environ)
    env.update(OXA_LIBRARY=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", CHILD], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
