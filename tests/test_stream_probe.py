"""The benchmark's streaming probes (librwkv_stream_probe.so): the bench line reports the
forward's and backward's traffic rates against wkv_stream_probe, and the decode's time
against wkv_stream_probe_decode, so both must compute what they claim. Shape checks run on
the CPU (they return before any GPU call); the arithmetic is checked on the GPU."""
import ctypes
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBE = os.path.join(ROOT, "rwkv_linear_attention_forward_amd", "librwkv_stream_probe.so")
NULL = ctypes.c_void_p(0)


def _lib():
    if not os.path.exists(PROBE):
        raise RuntimeError("%s is not built (python -c 'import __graft_entry__ as g; g.build()')"
                           % PROBE)
    return ctypes.CDLL(PROBE)


def _i64(x):
    return ctypes.c_int64(x)


def test_probe_exports_and_rejects_untiled_shapes():
    lib = _lib()
    dummy = ctypes.c_void_p(64)  # never dereferenced: every call below fails its shape check
    # layout ceiling: C a multiple of 64 * strips, R of 32 * chunks, layouts 1x2, 2x2, 4x1
    for R, C, strips, chunks in ((64, 96, 1, 2), (48, 64, 1, 2), (64, 192, 2, 2),
                                 (32, 128, 4, 1), (64, 64, 3, 1), (64, 64, 1, 1), (0, 64, 1, 2)):
        assert lib.wkv_stream_probe(_i64(R), _i64(C), dummy, dummy, dummy, strips, chunks, 0,
                                    NULL) == 1, (R, C, strips, chunks)
    assert lib.wkv_stream_probe(_i64(64), _i64(64), dummy, dummy, dummy, 1, 2, 65537, NULL) == 1
    assert lib.wkv_stream_probe(_i64(64), _i64(64), NULL, dummy, dummy, 1, 2, 0, NULL) == 1
    # decode ceiling: C a multiple of 256, B of 4, B / 4 <= 65535
    six = [dummy] * 6
    for B, C in ((4, 200), (6, 256), (0, 256), (4 * 65536, 256), (4, 0)):
        assert lib.wkv_stream_probe_decode(_i64(B), _i64(C), *six, NULL) == 1, (B, C)
    assert lib.wkv_stream_probe_decode(_i64(4), _i64(256), dummy, dummy, dummy, dummy, NULL,
                                       dummy, NULL) == 1


@pytest.mark.gpu
def test_layout_probe_writes_the_sum(dev):
    import torch
    lib = _lib()
    R, C = 256, 512
    k, v = torch.randn(R, C, device=dev), torch.randn(R, C, device=dev)
    for strips, chunks in ((1, 2), (2, 2), (4, 1)):
        y = torch.full_like(k, float("nan"))
        rc = lib.wkv_stream_probe(_i64(R), _i64(C), ctypes.c_void_p(k.data_ptr()),
                                  ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(y.data_ptr()),
                                  strips, chunks, 0,
                                  ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
        torch.cuda.synchronize()
        assert rc == 0
        assert torch.equal(y, k + v), (strips, chunks)


@pytest.mark.gpu
def test_decode_probe_updates_in_place(dev):
    import torch
    lib = _lib()
    B, C = 12, 768
    k, v, a, b, p = (torch.randn(B, C, device=dev) for _ in range(5))
    a0, b0, p0 = a.clone(), b.clone(), p.clone()
    y = torch.full_like(k, float("nan"))
    ptrs = [ctypes.c_void_p(t.data_ptr()) for t in (k, v, a, b, p, y)]
    rc = lib.wkv_stream_probe_decode(_i64(B), _i64(C), *ptrs,
                                     ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    torch.cuda.synchronize()
    assert rc == 0
    assert torch.equal(y, k + v)
    assert torch.equal(a, a0 + k) and torch.equal(b, b0 + v) and torch.equal(p, p0 + 1.0)
