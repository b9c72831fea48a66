"""Sanitizer builds on the CPU: the C oracle, and the host code of the HIP library (its device
code is built as usual), each linked with a small driver under tests/sanitize/ and run under
AddressSanitizer + UndefinedBehaviorSanitizer.  An out-of-bounds access or undefined arithmetic in
the oracle, or in the library's shape checks and workspace layout, aborts the driver."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "token_dispatch_grouped_route_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, env=ENV)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-2000:], r.stderr[-4000:])
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-Wall", "-Wno-unknown-pragmas", "-o", exe,
          os.path.join(HERE, "oracle_sanitize_main.c"), os.path.join(ROOT, "oracle", "moe_oracle.c"), "-lm"],
         str(tmp_path))
    assert "ok" in _run([exe], str(tmp_path))


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_library_host_code_under_address_and_undefined_sanitizers(tmp_path):
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC] + SAN_HOST
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    srcs.append(os.path.join(HERE, "abi_host_sanitize_main.cpp"))
    objs = [str(tmp_path / (os.path.basename(s) + ".o")) for s in srcs]
    with ThreadPoolExecutor(4) as pool:
        list(pool.map(lambda so: _run([HIPCC, *flags, "-c", so[0], "-o", so[1]], str(tmp_path)), zip(srcs, objs)))
    exe = str(tmp_path / "host_san")
    _run([HIPCC, "--offload-arch=gfx950", *SAN_HOST, "-o", exe, *objs], str(tmp_path))
    assert "ok" in _run([exe], str(tmp_path))
