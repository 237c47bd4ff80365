"""Build libdspark.so (HIP for gfx950) in-tree.

    python -m draft_sampling_verification_bias_amd.build

Compiles every source under ``csrc/`` with hipcc into ``_build/`` and links
``libdspark.so`` next to this file.  Always recompiles.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdspark.so")

ARCH = "gfx950"
SOURCES = ["api.cpp", "profile.cpp", "noalloc.hip", "tile_pass.hip", "draft.hip", "resident.hip", "verify.hip", "survival.hip", "weights.hip",
           "schedule.hip", "confidence.hip"]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build libdspark")


def _flags():
    return [
        "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
        "-I" + INCLUDE, "-I" + CSRC,
        # no packed-fp32 (v_pk_*_f32) code generation
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
    ]


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc()] + _flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), res.stderr))
    if verbose and res.stderr.strip():
        noise = "is not a recognized feature for this target"
        lines = [l for l in res.stderr.splitlines() if noise not in l]
        if lines:
            print("\n".join(lines), file=sys.stderr)
    return obj


def build(verbose=False):
    """Compile and link libdspark.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), res.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
