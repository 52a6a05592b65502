"""Build libsambay.so (the gfx950 HIP library) in-tree with hipcc.

    python attention_decoding_amd/build.py        # compile every csrc/*.hip, link

Objects go to _build/ at the repository root; the shared library is written
next to this file so that the Python binding (and a copy of the tree on a GPU
machine) finds it without installation.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build", "sambay")
LIB = os.path.join(PKG, "libsambay.so")
ARCH = os.environ.get("SAMBAY_OFFLOAD_ARCH", "gfx950")

# Packed-fp32 VALU forms are disabled for all device code.
COMMON_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I" + INCLUDE, "-I" + CSRC]


def source_hash() -> str:
    """First 16 hex digits of the SHA-256 of every kernel and header source
    (csrc/*.hip, csrc/*.hpp, include/*.h), names included; built into the
    library's version string so that a loaded binary can be tied to the
    sources it came from."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.hpp")) +
                   glob.glob(os.path.join(INCLUDE, "*.h")))
    for f in files:
        h.update(os.path.relpath(f, ROOT).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def hipcc() -> str:
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found (ROCm toolchain required to build libsambay.so)")
    return h


def _compile(src: str, extra) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [hipcc()] + COMMON_FLAGS + list(extra) + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(extra_flags=(), jobs: int | None = None, verbose: bool = False) -> str:
    """Compile all csrc/*.hip for gfx950 and link libsambay.so.  Always rebuilds."""
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    extra_flags = list(extra_flags) + ['-DSAMBAY_SOURCE_HASH="%s"' % source_hash()]
    jobs = jobs or min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra_flags), srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(extra_flags=sys.argv[1:], verbose=True)
