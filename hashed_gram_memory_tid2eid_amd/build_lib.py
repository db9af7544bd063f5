"""Build of libengram.so (gfx950) in-tree with hipcc.

Usage: ``python hashed_gram_memory_tid2eid_amd/build_lib.py`` (run by path: importing
the package loads the library this script builds).  Compiles the single
device translation unit and the host sources to objects under ``_build/`` and
links ``hashed_gram_memory_tid2eid_amd/libengram.so``.  Always recompiles.

The library carries a hash of what it was built from (every source under
``csrc/`` and ``include/`` plus the compiler flags), readable with
``engram_build_id()``.  ``ensure_built()`` rebuilds whenever that hash differs
from the sources in the tree, so a stale library is never loaded.
"""
from __future__ import annotations

import hashlib
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libengram.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops stay off: the compiler's own scalar/float2 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include"),
]

SOURCES = ["engram_device.hip", "abi.cpp", "layout.cpp", "noalloc.cpp"]
INCLUDE = os.path.join(ROOT, "include")
BUILD_ID_PREFIX = "engram-src-sha256:"


def source_hash() -> str:
    """First 16 hex digits of a SHA-256 over every source file under csrc/ and
    include/ (relative path and bytes, in sorted order) and the compiler flags (paths
    inside the tree written relative to it)."""
    h = hashlib.sha256()
    for top in (CSRC, INCLUDE):
        for root, dirs, files in os.walk(top):
            dirs.sort()
            for f in sorted(files):
                if f.endswith((".hip", ".cpp", ".h", ".hpp", ".inc")):
                    path = os.path.join(root, f)
                    h.update(os.path.relpath(path, ROOT).encode())
                    with open(path, "rb") as fh:
                        h.update(fh.read())
    # the flags with the tree's own location taken out, so a copy of the tree elsewhere
    # (same sources, same flags) keeps the identity and its built library
    h.update(" ".join(COMMON).replace(ROOT, ".").encode())
    return h.hexdigest()[:16]


def built_hash(lib: str = LIB):
    """The source hash recorded in a built library, or None (missing, or built
    before the hash existed)."""
    if not os.path.exists(lib):
        return None
    with open(lib, "rb") as f:
        m = re.search(re.escape(BUILD_ID_PREFIX.encode()) + rb"([0-9a-f]{16})", f.read())
    return m.group(1).decode() if m else None


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    sha = source_hash()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"]
        defs = [f'-DENGRAM_BUILD_ID="{BUILD_ID_PREFIX}{sha}"'] if src == "abi.cpp" else []
        cmd = [HIPCC, *COMMON, *defs, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the device-only target feature; that warning is noise
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
        if p.returncode != 0:
            failed.append(src)
            print(text, file=sys.stderr)
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


MFMA_CEILING_SRC = os.path.join(PKG, "calibrate", "mfma_ceiling.hip")
MFMA_CEILING_BIN = os.path.join(BUILD, "mfma_ceiling")


def build_mfma_ceiling() -> str:
    """Builds the matrix-core ceiling probe (a measurement program beside the
    library, run by `bench.py --mfma-ceiling`) and returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    cmd = [HIPCC, *COMMON, MFMA_CEILING_SRC, "-o", MFMA_CEILING_BIN]
    out = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if out.returncode != 0:
        print(out.stdout.decode(errors="replace"), file=sys.stderr)
        raise RuntimeError("hipcc failed for the matrix-core ceiling probe")
    return MFMA_CEILING_BIN


HBM_REFERENCE_SRC = os.path.join(PKG, "calibrate", "hbm_reference.hip")
HBM_REFERENCE_BIN = os.path.join(BUILD, "hbm_reference")


def build_hbm_reference() -> str:
    """Builds the HBM streaming-reference probe (a measurement program beside the
    library, run by `bench.py --hbm-reference`) and returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    cmd = [HIPCC, *COMMON, HBM_REFERENCE_SRC, "-o", HBM_REFERENCE_BIN]
    out = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if out.returncode != 0:
        print(out.stdout.decode(errors="replace"), file=sys.stderr)
        raise RuntimeError("hipcc failed for the HBM reference probe")
    return HBM_REFERENCE_BIN


def ensure_built() -> str:
    """Builds the library when it is missing or was built from other sources than
    the tree holds now (compared by the embedded source hash); otherwise leaves
    the built one in place."""
    if built_hash() == source_hash():
        return LIB
    return build()


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
