"""Register budgets of the hot kernels, from the compiler's resource report (CPU only).

The streaming kernels are latency-bound chains over HBM: the forward and backward keep
three waves per SIMD only while they fit in 168 VGPRs, and losing the third wave costs
them about a quarter of their speed. A small change far from the hot loop (a 64-bit
division in a one-thread branch, a value loaded late in a branch) can push the whole
kernel's allocation past that line, so each hot instance's budget is checked here on
every change: hipcc compiles the sources for gfx950 with the build's own flags and
reports VGPRs, spills and occupancy per kernel.
"""
import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "rwkv_linear_attention_forward_amd")
CSRC = os.path.join(PKG, "csrc")


def _report(src, tmp_path):
    sys.path.insert(0, PKG)
    try:
        import build
    finally:
        sys.path.pop(0)
    cmd = [build.HIPCC] + build.FLAGS + ["-Rpass-analysis=kernel-resource-usage", "-c",
                                         os.path.join(CSRC, src), "-o",
                                         str(tmp_path / (src + ".o"))]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out = {}
    for block in re.split(r"remark: [^\n]*Function Name: ", r.stderr)[1:]:
        name = block.split()[0]
        out[name] = {k: int(re.search(k + r": (\d+)", block).group(1))
                     for k in ("VGPRs", "VGPRs Spill")}
        out[name]["occupancy"] = int(re.search(r"Occupancy \[waves/SIMD\]: (\d+)", block).group(1))
    return out


@pytest.fixture(scope="module")
def reports(tmp_path_factory):
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    tmp = tmp_path_factory.mktemp("res")
    srcs = ("wkv_forward.hip", "wkv_backward.hip", "wkv_decode.hip")
    with ThreadPoolExecutor(max_workers=3) as ex:
        return dict(zip(srcs, ex.map(lambda s: _report(s, tmp), srcs)))


def _instances(rep, needle):
    got = {n: v for n, v in rep.items() if needle in n}
    assert got, "no %s instance in the report" % needle
    return got


def test_forward_keeps_three_waves_per_simd(reports):
    for name, r in _instances(reports["wkv_forward.hip"], "wkv_forward_kernel").items():
        assert r["occupancy"] >= 3 and r["VGPRs Spill"] == 0, (name, r)


def test_backward_keeps_three_waves_per_simd(reports):
    for name, r in _instances(reports["wkv_backward.hip"], "wkv_backward_kernel").items():
        gated = re.search(r"ILi2ELi32ELb1E", name) is not None
        assert r["occupancy"] >= 3, (name, r)
        assert r["VGPRs Spill"] <= (2 if gated else 0), (name, r)


def test_small_kernels_stay_light(reports):
    for name, r in _instances(reports["wkv_backward.hip"], "wkv_reduce_kernel").items():
        assert r["occupancy"] >= 8, (name, r)
    for name, r in _instances(reports["wkv_decode.hip"], "wkv_decode_kernel").items():
        assert r["occupancy"] >= 8 and r["VGPRs Spill"] == 0, (name, r)
