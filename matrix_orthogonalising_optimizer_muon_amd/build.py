"""Build ``libmuon_amd.so`` (HIP for gfx950) in-tree with hipcc.

Usage: ``python -m matrix_orthogonalising_optimizer_muon_amd.build`` (or
``__graft_entry__.build()``). Objects go to ``_build/``; the library lands next to this
file, where the binding loads it.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build", "muon_amd")
LIB = os.path.join(PKG, "libmuon_amd.so")
SOURCES = ["api.cpp", "gemm.hip", "elementwise.hip", "small.hip", "adamw.hip", "planner.cpp"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-x", "hip",
    "-Wall", "-Wno-unused-function",
    # packed fp32 arithmetic is kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str, verbose: bool) -> str:
    out = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)  # host pass does not know the feature
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if verbose and msg.strip():
        print(msg, flush=True)
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the C++ front end (argument
# validation, planning, tune-file parsing, owner planner) for the host-only tests. Device
# code is built as usual (sanitizers apply to the host pass only); the kernels' objects of
# the regular build are reused when they are newer than their sources.
SAN_OBJ = os.path.join(ROOT, "_build", "asan")
SAN_LIB = os.path.join(SAN_OBJ, "libmuon_amd_asan.so")
SAN_SOURCES = ["api.cpp", "planner.cpp"]
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def asan_runtime() -> str | None:
    """The clang AddressSanitizer runtime to preload into an uninstrumented Python."""
    import glob
    root = os.path.dirname(os.path.dirname(os.path.realpath(HIPCC)))
    hits = sorted(glob.glob(os.path.join(root, "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    hits += sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[0] if hits else None


def build_asan(verbose: bool = False) -> str:
    os.makedirs(SAN_OBJ, exist_ok=True)

    def obj(src):
        if src in SAN_SOURCES:
            out = os.path.join(SAN_OBJ, os.path.splitext(src)[0] + ".o")
            cmd = [HIPCC, *[f for f in FLAGS if f != "-O3"], "-O1", "-g", *SAN_FLAGS, "-c",
                   os.path.join(CSRC, src), "-o", out]
        else:
            out = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
            if os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(os.path.join(CSRC, src)):
                return out
            os.makedirs(OBJ, exist_ok=True)
            cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", out]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}{r.stderr}")
        return out

    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(obj, SOURCES))
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libasan", "-Xarch_host",
           "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", *objs, "-o", SAN_LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    return SAN_LIB


if __name__ == "__main__":
    if "--asan" in sys.argv:
        print(build_asan(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
