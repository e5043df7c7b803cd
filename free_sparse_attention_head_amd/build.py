"""Build libfsa.so (the C-ABI HIP library) in-tree for gfx950.

    python -m free_sparse_attention_head_amd.build                 # both libraries
    python -m free_sparse_attention_head_amd.build --release-only  # libfsa.so
    python -m free_sparse_attention_head_amd.build --debug-bounds  # libfsa_debug.so

Every HIP translation unit is compiled with hipcc for --offload-arch=gfx950 in
parallel, then linked into free_sparse_attention_head_amd/libfsa.so.  Packed
fp32 VALU instructions are disabled for device code.  The debug-bounds build
(-DFSA_DEBUG_BOUNDS) records the bad inputs the kernels skip, readable with
fsa_debug_flags (include/fsa.h); it is otherwise the same library.
"""

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfsa.so")
DEBUG_LIB = os.path.join(PKG, "libfsa_debug.so")
ARCH = "gfx950"


def _hipcc():
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return h


COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src, build_dir, extra):
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [_hipcc()] + COMMON + extra + ["-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [_hipcc(), "-x", "hip"] + COMMON + extra + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(x for x in r.stderr.splitlines() if noise not in x)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    return obj, err


def build(verbose=False, debug_bounds=False):
    """Compile every source and link libfsa.so (libfsa_debug.so with
    debug_bounds); returns the library path."""
    build_dir = BUILD_DIR + ("_debug" if debug_bounds else "")
    lib = DEBUG_LIB if debug_bounds else LIB
    extra = ["-DFSA_DEBUG_BOUNDS"] if debug_bounds else []
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "fsa_api.cpp")]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(lambda x: _compile(x, build_dir, extra), srcs))
    for obj, err in results:
        if verbose and err.strip():
            print(err, file=sys.stderr)
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    if "--debug-bounds" not in sys.argv:
        print(build(verbose=True))
    if "--release-only" not in sys.argv:
        print(build(verbose=True, debug_bounds=True))
