"""Process-level checks on the GPU (marked gpu): the library runs on gfx950 and
shares the single HIP runtime that torch loaded."""
import pytest

pytestmark = pytest.mark.gpu


def test_single_hip_runtime_and_gfx950(wkv, dev):
    import torch
    x = torch.zeros(1, 4, 8, device=dev)
    w = torch.ones(8, device=dev)
    wkv.forward(w, w, x, x)
    torch.cuda.synchronize()
    maps = open("/proc/self/maps").read().split("\n")
    hip = sorted({l.split()[-1] for l in maps if "libamdhip64" in l})
    print("[runtime] HIP runtimes mapped:", hip, flush=True)
    assert len(hip) == 1, hip
    assert "gfx950" in torch.cuda.get_device_properties(0).gcnArchName
    assert any("librwkv_wkv.so" in l for l in maps)
