"""Build liboxa.so (the C-ABI library with the gfx950 kernels) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liboxa.so")
SOURCES = ["decode.hip", "decode_balanced.hip", "append.hip", "prefill.hip", "merge.hip", "rope.hip", "oxa_host.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed-FP32 VALU forms are kept out of the generated code on purpose.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the GPU-only feature flag; that warning is noise
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed: {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False, jobs: int = 4) -> str:
    os.makedirs(BUILD, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(BUILD, src + ".o")
        out = _run([HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and out.strip():
            print(out, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


HOST_SANITIZED = os.path.join(BUILD, "liboxa_host_sanitized.so")


def build_host_sanitized(jobs: int = 4) -> str:
    """liboxa with its host layer (argument checks, workspace layout, launch
    set-up) built under AddressSanitizer and UndefinedBehaviorSanitizer, host
    pass only; the kernels are the regular objects.  For CPU tests of the host
    layer: load it with the ASan runtime preloaded (see the host sanitizer test)."""
    objs = []
    missing = [s for s in SOURCES if s != "oxa_host.cpp" and
               not os.path.exists(os.path.join(BUILD, s + ".o"))]
    if missing:
        build(jobs=jobs)
    for src in SOURCES:
        if src != "oxa_host.cpp":
            objs.append(os.path.join(BUILD, src + ".o"))
    obj = os.path.join(BUILD, "oxa_host_sanitized.o")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
           "-g"]
    _run([HIPCC, *FLAGS, *san, "-c", os.path.join(CSRC, "oxa_host.cpp"), "-o", obj])
    # the sanitizer runtime is not linked in: the process preloads it
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", obj, *objs, "-o", HOST_SANITIZED])
    return HOST_SANITIZED


if __name__ == "__main__":
    print(build(verbose=True))
