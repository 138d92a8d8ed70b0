"""The CPU oracle and the library's host side under AddressSanitizer and
UndefinedBehaviorSanitizer (no GPU): each is built with the sanitizers into
a harness executable (tests/sanitize/) and run; any memory error or
undefined behaviour aborts it.

  * oracle: oracle.c with gcc, driven on small seeded inputs through every
    function, degenerate cases included (leak checking on);
  * host side: every library source compiled with hipcc as for the library
    (gfx950 device code, packed fp32 off) with the sanitizers on the host
    pass only, driven through every C-ABI call's argument validation and
    host arithmetic (workspace and plan sizes, status text, switches), with
    arguments the validation refuses before any HIP call -- so no GPU is
    needed or touched.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "moe_block_skinny_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-3000:], r.stderr[-6000:])
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_harness")
    _run(["gcc", "-std=c11", "-ffp-contract=off"] + SAN +
         [os.path.join(HERE, "oracle_harness.c"), os.path.join(ROOT, "oracle", "oracle.c"), "-lm", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = _run([exe], env=env)
    assert "0 failures" in r.stdout


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not found")
def test_host_side_under_asan_ubsan(tmp_path):
    cc = _hipcc()
    # the sanitizers go to the host pass only; no device code is built
    host_san = []
    for f in SAN:
        host_san += ["-Xarch_host", f] if f.startswith("-fsanitize") or f.startswith("-fno-sanitize") else [f]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))

    dev = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([cc, "-std=c++17", "-fPIC"] + dev + host_san + inc + ["-c", src, "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(compile_one, srcs + [os.path.join(HERE, "host_harness.cpp")]))
    exe = str(tmp_path / "host_harness")
    _run([cc, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address,undefined"] + objs + ["-o", exe])
    # the HIP runtime library is loaded but never called; its own start-up
    # allocations are not this code's, so leak checking is off here
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = _run([exe], env=env)
    assert "0 failures" in r.stdout
