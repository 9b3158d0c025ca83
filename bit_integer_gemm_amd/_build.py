"""Build the gfx950 shared library ``liblbgemm.so`` in-tree with hipcc.

Usage: ``python -m bit_integer_gemm_amd._build`` (or ``build()`` from Python).
Every HIP/C++ source under ``csrc/`` is compiled for gfx950 only and linked
into one library exporting the C ABI of ``include/lb_gemm.h``.

``python -m bit_integer_gemm_amd._build --ab NAME`` builds an A/B profiling
library instead, ``bit_integer_gemm_amd/ab/liblbgemm_NAME.so``, with one design
choice turned off (see AB_BUILDS); ``bench.py --lib`` loads it.  The library the
package uses is never built that way.
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liblbgemm.so")
OBJDIR = os.path.join(PKG, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    # packed fp32 VALU ops are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Werror", "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


# A/B profiling builds: one design choice of the kernels turned off each
# (the macros are documented in csrc/lb_mfma.hip and csrc/lb_device.hpp).
AB_BUILDS = {
    "no_swizzle": ["-DLB_AB_LDS_SWIZZLE=0"],
    "rows_spread": ["-DLB_AB_COPY_ROWS_SPREAD=1"],
    "plain_tile_map": ["-DLB_AB_TILE_MAP_PLAIN=1"],
    "copy_burst": ["-DLB_AB_COPY_BURST=1"],
    "w4_int8_only": ["-DLB_AB_W4_INT8_ONLY=1"],
    "w4_bands": ["-DLB_AB_W4_BANDS=1"],
    "reg_staging": ["-DLB_AB_REG_STAGING=1"],
}
AB_DIR = os.path.join(PKG, "ab")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def source_files():
    """Every file the library is built from: the sources, their headers and
    generated tables under csrc/, and the public header."""
    files = [os.path.join(CSRC, f) for f in os.listdir(CSRC)
             if f.endswith((".hip", ".cpp", ".hpp", ".inc"))]
    files.append(os.path.join(INCLUDE, "lb_gemm.h"))
    return sorted(files)


def source_sha() -> str:
    """Hash of the exact text of every source file (16 hex digits).  The build
    stamps it into the library, which returns it from lb_build_id(), so that a
    loaded library can be matched with the sources it was built from."""
    h = hashlib.sha256()
    for f in source_files():
        h.update(os.path.relpath(f, ROOT).encode())
        h.update(b"\0")
        with open(f, "rb") as fh:
            h.update(fh.read())
        h.update(b"\0")
    return h.hexdigest()[:16]


_MARK = re.compile(rb"lb-source-sha:([0-9a-f]{16})")


def built_sha(path: str = None):
    """The source hash stamped into a built library file (read from its bytes,
    without loading it), or None if there is no library or no stamp."""
    path = path or LIB
    if not os.path.exists(path):
        return None
    with open(path, "rb") as fh:
        m = _MARK.search(fh.read())
    return m.group(1).decode() if m else None


def ensure_built(verbose: bool = False) -> str:
    """Build the library when it is missing or was built from other sources."""
    if built_sha() != source_sha():
        build(verbose=verbose)
    return LIB


def _compile(src: str, sha: str, objdir: str = OBJDIR, defines=()) -> str:
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, f'-DLB_SOURCE_SHA="{sha}"', *defines, "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr[-6000:]}")
    return obj


def build(verbose: bool = False, ab: str = None) -> str:
    lib, objdir, defines = LIB, OBJDIR, ()
    if ab is not None:
        if ab not in AB_BUILDS:
            raise ValueError(f"unknown A/B build {ab!r}; choose from {sorted(AB_BUILDS)}")
        lib = os.path.join(AB_DIR, f"liblbgemm_{ab}.so")
        objdir = os.path.join(OBJDIR, "ab_" + ab)
        defines = tuple(AB_BUILDS[ab])
        os.makedirs(AB_DIR, exist_ok=True)
    os.makedirs(objdir, exist_ok=True)
    srcs = sources()
    sha = source_sha()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda f: _compile(f, sha, objdir, defines), srcs))
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-6000:]}")
    os.replace(tmp, lib)
    if built_sha(lib) != sha:
        raise RuntimeError(f"{lib} does not carry the source hash {sha}")
    if verbose:
        print(f"built {lib} (sources {sha}{', A/B ' + ab if ab else ''})")
    return lib


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("--ab", choices=sorted(AB_BUILDS), help="build an A/B profiling library instead")
    a = ap.parse_args()
    build(verbose=True, ab=a.ab)
    sys.exit(0)
