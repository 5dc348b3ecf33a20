"""Host code under AddressSanitizer and UBSan (CPU only).

Builds the C-ABI validation layer (`vpe_api.cpp`) against host stand-ins for
the kernel launchers, together with the CPU oracle, with g++/gcc and
`-fsanitize=address,undefined -fno-sanitize-recover=all`, and runs a driver
that exercises every entry point's accept and reject paths (edge and
overflow-prone sizes and offsets) and the oracle's loops on small heap
buffers.  No GPU code is built with a sanitizer.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


def _run(cmd):
    return subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)


def test_validation_layer_and_oracle_under_asan_ubsan():
    if shutil.which("g++") is None or shutil.which("gcc") is None:
        pytest.skip("no host compiler")
    with tempfile.TemporaryDirectory() as tmp:
        objs = []
        for src, cc, extra in [
                (os.path.join(HERE, "driver.cpp"), "g++", ["-std=c++17", "-I", os.path.join(ROOT, "include")]),
                (os.path.join(HERE, "stub_launchers.cpp"), "g++", ["-std=c++17"]),
                (os.path.join(ROOT, "vocab_sharded_embedding_amd", "csrc", "vpe_api.cpp"), "g++",
                 ["-std=c++17"]),
                (os.path.join(ROOT, "oracle", "oracle.c"), "gcc", ["-std=c11", "-ffp-contract=off"])]:
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            r = _run([cc, *extra, *SAN, "-c", src, "-o", obj])
            if r.returncode != 0 and "asan" in r.stdout.lower():
                pytest.skip("sanitizer runtime not available: " + r.stdout[-300:])
            assert r.returncode == 0, r.stdout
            objs.append(obj)
        exe = os.path.join(tmp, "host_sanitize")
        r = _run(["g++", *SAN, *objs, "-lpthread", "-o", exe])
        assert r.returncode == 0, r.stdout
        r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                           env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0"})
        assert r.returncode == 0, r.stdout
        assert "all expectations held" in r.stdout
