"""Build libhtl.so (the C-ABI HIP library) in-tree for gfx950.

Each HIP source compiles to an object in parallel, then hipcc links the
shared library next to this file.  Usage: ``python -m hash_table_lookup_amd.build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libhtl.so")
ARCH = os.environ.get("HTL_OFFLOAD_ARCH", "gfx950")

SOURCES = ["table.hip", "dedup.hip", "lookup.hip", "gather.hip", "pool.hip", "scan.hip", "backward.hip", "lru.hip",
           "copy.hip", "noalloc.hip", "debug.hip"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-function",
    # keep the compiler from forming packed-fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return p


# Host code built with AddressSanitizer and UndefinedBehaviorSanitizer (the
# device code is built as usual): a library for checking the host side --
# argument checks, workspace layouts, table bookkeeping -- under the
# sanitizers, loaded in place of libhtl.so through HTL_LIB with the clang
# ASan runtime preloaded.
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
SAN_BUILD_DIR = os.path.join(HERE, "_build_san")
SAN_LIB_PATH = os.path.join(HERE, "libhtl_san.so")
# debug build: the same kernels plus device-side invariant checks after each
# find-or-insert, dedup and logged erase (htl_debug_flags reads what they
# found), loaded in place of libhtl.so through HTL_LIB
DEBUG_BUILD_DIR = os.path.join(HERE, "_build_dbg")
DEBUG_LIB_PATH = os.path.join(HERE, "libhtl_debug.so")


def _compile(src: str, san: bool = False, debug: bool = False) -> str:
    out_dir = SAN_BUILD_DIR if san else (DEBUG_BUILD_DIR if debug else BUILD_DIR)
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    flags = [f for f in HIPCC_FLAGS if not (san and f == "-O3")] + (["-O1", "-g"] + SAN_FLAGS if san else [])
    if debug:
        flags = flags + ["-DHTL_DEBUG"]
    cmd = [_hipcc(), *flags, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 8, verbose: bool = True, sanitize: bool = False, debug: bool = False) -> str:
    """Compile every HIP source and link libhtl.so (sanitize: libhtl_san.so,
    host code under ASan + UBSan; debug: libhtl_debug.so, with the device-side
    invariant checks); returns its path."""
    if sanitize:
        out_dir, lib = SAN_BUILD_DIR, SAN_LIB_PATH
    elif debug:
        out_dir, lib = DEBUG_BUILD_DIR, DEBUG_LIB_PATH
    else:
        out_dir, lib = BUILD_DIR, LIB_PATH
    os.makedirs(out_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(SOURCES)))) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize, debug), SOURCES))
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if sanitize:
        cmd[3:3] = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libasan"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    args = [a for a in sys.argv[1:] if a not in ("--sanitize", "--debug")]
    build(jobs=int(args[0]) if args else 8, sanitize="--sanitize" in sys.argv, debug="--debug" in sys.argv)
