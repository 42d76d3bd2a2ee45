"""Build libkvscore.so (the HIP kernels + C ABI) for gfx950, in-tree.

Usage: python -m kv_cache_eviction_amd.build [-v] [--sanitize]
Each source compiles to an object under kv_cache_eviction_amd/_build/, then
they link into kv_cache_eviction_amd/libkvscore.so.  Always rebuilds.

--sanitize builds kv_cache_eviction_amd/_build_san/libkvscore.so with the
host code (argument checks, workspace planning, dispatch) instrumented by
AddressSanitizer and UndefinedBehaviorSanitizer; the device code is built as
usual.  The sanitizer runtime is not linked in: load it first with
LD_PRELOAD (see README), and select this library with KVS_SANITIZED_BUILD=1.
"""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkvscore.so")
BUILD_SAN = os.path.join(PKG, "_build_san")
LIB_SAN = os.path.join(BUILD_SAN, "libkvscore.so")
# host-only sanitizer flags: each -fsanitize= right after -Xarch_host, so the
# device code is compiled exactly as in the normal build
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
SOURCES = ["attn.hip", "deletion.hip", "select.hip", "h2o.hip", "reliability.hip", "fidelity.hip", "peaks.hip", "prefill.hip",
           "timing.cpp",
           "capi.cpp"]
ARCH = "gfx950"


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libkvscore.so)")


def _flags():
    return ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "--offload-arch=" + ARCH,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # MFMA results in VGPRs: the epilogues read them with ordinary VALU
            # operands instead of one accvgpr read per element
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-Wno-unused-command-line-argument"]


def _compile(src, verbose, sanitize=False):
    obj = os.path.join(BUILD_SAN if sanitize else BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc()] + _flags() + (SAN_FLAGS if sanitize else []) + [
        "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError("compiling %s failed:\n%s" % (src, msg))
    if verbose and msg:
        print(msg, flush=True)
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    os.makedirs(BUILD_SAN if sanitize else BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, sanitize), SOURCES))
    lib = LIB_SAN if sanitize else LIB
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("linking libkvscore.so failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
