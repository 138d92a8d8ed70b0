"""Build the gfx950 shared library libmoe_skinny.so in-tree with hipcc.

    python -m moe_block_skinny_amd.build [--stamps]

Every .hip / .cpp file under csrc/ is compiled for gfx950 only (no other
target, no CUDA path) and linked into one C-ABI shared library.  All device
code is built with packed-fp32 instructions disabled.  With stamps=True the
same sources are built with -DMOE_STAMPS into libmoe_skinny_stamps.so: the
instrumented library whose kernels record per-workgroup clock stamps
(`bench.py --timeline`); nothing else loads it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe_skinny.so")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_STAMPS = os.path.join(HERE, "libmoe_skinny_stamps.so")
BUILD_DIR_STAMPS = os.path.join(HERE, "_build_stamps")

ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def flags() -> list:
    return [
        "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    ]


def sources() -> list:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def source_digest() -> str:
    """sha256 over the sources of the kernels and their launches (csrc/), so
    a stored profile can tell whether the kernels changed since it was taken
    (the public header only declares, so its comments may change freely)."""
    import hashlib
    h = hashlib.sha256()
    files = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp", ".hpp")))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def build(verbose: bool = False, stamps: bool = False) -> str:
    bdir, lib = (BUILD_DIR_STAMPS, LIB_STAMPS) if stamps else (BUILD_DIR, LIB)
    os.makedirs(bdir, exist_ok=True)
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(bdir, os.path.basename(src) + ".o")
        cmd = [cc] + flags() + (["-DMOE_STAMPS"] if stamps else []) + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError("compile failed: %s\n%s" % (src, err))
        if err.strip() and verbose:
            print(err, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(compile_one, sources()))
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [cc, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, stamps="--stamps" in sys.argv))
