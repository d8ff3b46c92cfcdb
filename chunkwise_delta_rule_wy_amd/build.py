"""Build the HIP library ``libdn.so`` for gfx950 with hipcc (in-tree)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdn.so")
# the machine probes of the benchmark (measured MFMA rate, shader clock) live in a
# library of their own
PROBE_LIB = os.path.join(HERE, "libdnprobe.so")
PROBE_SOURCES = ["dn_probe.hip"]
# per-source flags: the probe's MFMA loop keeps its accumulators in VGPRs (with
# AGPR accumulators the register allocator shuffles them between rounds)
EXTRA_FLAGS = {"dn_probe.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
SOURCES = ["dn_api.hip", "dn_fwd.hip", "dn_fwd32.hip", "dn_fwd_f32.hip", "dn_bwd.hip", "dn_scan.hip", "dn_bwd_chunk.hip", "dn_step.hip", "dn_longhorn.hip", "dn_prologue.hip", "dn_conv.hip", "dn_noalloc.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    p = os.path.join(rocm, "bin", "hipcc")
    return p if os.path.exists(p) else "hipcc"


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libdn.so (and libdnprobe.so) next to
    this file."""
    _link(SOURCES, LIB, verbose)
    _link(PROBE_SOURCES, PROBE_LIB, verbose)
    return LIB


def _compile(src, objdir):
    obj = os.path.join(objdir, src.replace(".hip", ".o"))
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    cmd = [_hipcc()] + HIPCC_FLAGS + EXTRA_FLAGS.get(src, []) + inc + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines()
                    if "not a recognized feature" not in ln)
    return obj, r.returncode, msg


def _link(sources, lib, verbose):
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    jobs = max(1, min(len(sources), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1)), 16))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, objdir), sources))
    objs = []
    for src, (obj, rc, msg) in zip(sources, results):
        if rc != 0:
            raise RuntimeError("hipcc failed for %s:\n%s" % (src, msg))
        if verbose and msg.strip():
            print(msg, file=sys.stderr)
        objs.append(obj)
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s%s" % (r.stdout, r.stderr))
    os.replace(tmp, lib)


if __name__ == "__main__":
    print(build(verbose=True))
