"""Build librwkv_wkv.so (and the benchmark's librwkv_stream_probe.so) in-tree with hipcc for
gfx950.

Every .hip file under csrc/ is compiled to an object in _build/ (in parallel) and the
objects are linked into rwkv_linear_attention_forward_amd/librwkv_wkv.so. The build
always recompiles: it is the "does it build" check as well as the build.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "librwkv_wkv.so")
# the benchmark's streaming-ceiling probe: a library of its own, not part of the operator's
PROBE_SRC = os.path.join(PKG, "probe", "stream_probe.hip")
PROBE_LIB = os.path.join(PKG, "librwkv_stream_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep hipcc from forming v_pk_{add,mul,fma}_f32 out of scalar fp32 code.
# -ffp-contract=off: fused multiply-adds only where the source writes fma(), so that the same
# expression gives the same bits wherever it is inlined (a look-back helper must reproduce
# a unit's published summary exactly).
# The host pass prints that it does not know the feature; that warning is harmless.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-mcode-object-version=5",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (src, out))
    if out.strip():
        sys.stderr.write(out + "\n")
    return obj


def build(jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    build_probe()
    return LIB


def build_probe() -> str:
    """librwkv_stream_probe.so (bench.py's layout-ceiling leg)."""
    os.makedirs(BUILD, exist_ok=True)
    tmp = PROBE_LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-shared", PROBE_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (PROBE_SRC, r.stdout + r.stderr))
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    print(build())
