"""Build libvpe.so in-tree: HIP kernels for gfx950 with hipcc, the C-ABI layer
with g++ (it has no HIP dependency), linked into one shared library."""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import subprocess
import sys
from typing import List

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libvpe.so")
DIGEST = LIB + ".sha256"  # digest of the sources and flags the library was built from
OBJDIR = os.path.join(PKG, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HIP_SOURCES = ["gather.hip", "lmhead.hip"]
CXX_SOURCES = ["vpe_api.cpp"]

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    # packed fp32 instructions stay off: hipcc only emits plain fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]
CXX_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-Wall", "-Wextra", "-I", INCLUDE, "-I", CSRC]


def source_files() -> List[str]:
    """Every file the library is built from: kernels, the C-ABI layer, the
    internal headers, the public header and build.py itself."""
    names = sorted(f for f in os.listdir(CSRC)
                   if f.endswith((".hip", ".cpp", ".h")))
    return [os.path.join(CSRC, f) for f in names] + [os.path.join(INCLUDE, "vpe.h"),
                                                     os.path.abspath(__file__)]


def source_digest() -> str:
    """sha256 over the names and contents of source_files()."""
    h = hashlib.sha256()
    for path in source_files():
        with open(path, "rb") as f:
            data = f.read()
        h.update(os.path.basename(path).encode() + b"\0" + str(len(data)).encode() + b"\0")
        h.update(data)
    return h.hexdigest()


def built_digest(lib: str = LIB) -> str:
    """The digest recorded next to a built library ('' when none is)."""
    try:
        with open(lib + ".sha256") as f:
            return f.read().strip()
    except OSError:
        return ""


def _run(cmd: List[str]) -> None:
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so: harmless
    lines = [l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l]
    if r.returncode != 0:
        sys.stderr.write("\n".join(lines) + "\n")
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}")
    if lines:
        sys.stderr.write("\n".join(lines) + "\n")


def build(verbose: bool = False) -> str:
    """Compile every source and link libvpe.so; returns the library path."""
    os.makedirs(OBJDIR, exist_ok=True)
    digest = source_digest()  # taken before compiling: a later edit makes it stale
    jobs = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(OBJDIR, src + ".o")
        jobs.append([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in CXX_SOURCES:
        obj = os.path.join(OBJDIR, src + ".o")
        jobs.append(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with cf.ThreadPoolExecutor(max_workers=min(len(jobs), 8)) as ex:
        for f in [ex.submit(_run, j) for j in jobs]:
            f.result()
    tmp = LIB + ".tmp%d" % os.getpid()
    # --no-undefined: a kernel whose host launch stub was not emitted fails here,
    # not at load time
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", *objs,
          "-o", tmp])
    os.replace(tmp, LIB)
    with open(DIGEST + ".tmp", "w") as f:
        f.write(digest + "\n")
    os.replace(DIGEST + ".tmp", DIGEST)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
