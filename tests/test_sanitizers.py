"""Host code under the address and undefined-behaviour sanitizers (no GPU).

1. The C ABI's host side (argument validation, workspace layout, parameter
   packing: csrc/dn_api.hip compiled for the host only) with the kernel
   launchers replaced by counting stand-ins, driven through every entry point
   with valid, invalid and extreme arguments (tests/sanitize/abi_validation.cpp).
2. The fp64 oracle (oracle/dn_oracle.c) on small fixed and packed inputs
   (tests/sanitize/oracle_main.c).

Any sanitizer report aborts the program and fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "chunkwise_delta_rule_wy_amd", "csrc")
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
# host-only compilation: each sanitizer flag is scoped to the host pass
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    out = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines() if "not a recognized feature" not in ln)
    assert r.returncode == 0, "%s\n%s" % (" ".join(cmd), out)
    return out


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_abi_host_validation_under_sanitizers(tmp_path):
    common = [HIPCC, "--offload-host-only", "-O1", "-g", "-std=c++17"] + HOST_SAN + [
        "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = []
    for src, lang in ((os.path.join(CSRC, "dn_api.hip"), []),
                      (os.path.join(SAN, "launch_stubs.cpp"), ["-x", "hip"]),
                      (os.path.join(SAN, "abi_validation.cpp"), ["-x", "hip"])):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run(common + lang + ["-c", src, "-o", obj])
        objs.append(obj)
    exe = str(tmp_path / "abi_validation")
    _run([HIPCC] + HOST_SAN[:4] + objs + ["-o", exe])
    out = _run([exe], env=ENV, timeout=120)
    assert "checks passed" in out, out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    _run(["gcc", "-O1", "-g", "-std=c99", "-fopenmp", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-o", exe, os.path.join(SAN, "oracle_main.c"),
          os.path.join(ROOT, "oracle", "dn_oracle.c"), "-lm"])
    out = _run([exe], env=ENV, timeout=300)
    assert "oracle sanitize: ok" in out, out
