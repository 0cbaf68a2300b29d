"""wkv_forward_noalloc, the forward for callers that cannot allocate (marked gpu).

Called through the C ABI twice in a row, the second time with a smaller input, it must give
bitwise the y of wkv_forward (the same scan, its scratch in the library's per-GPU array
instead of the stream-ordered pool) and y within the stated tolerance of the fp64 oracle.
The first call is the 3B-class layer, whose scratch nearly fills the array; the second
leaves the first call's records behind in it, which the per-call epochs must ignore.
"""
import ctypes

import numpy as np
import pytest

import oracle
import wkv_inputs
from helpers import assert_wkv_close

pytestmark = pytest.mark.gpu


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def test_noalloc_forward_matches_the_plain_forward(wkv, dev):
    import torch
    lib = wkv.load_library()
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    for (B, T, C, seed) in ((8, 4096, 2560, 41), (2, 300, 130, 42)):
        assert lib.wkv_forward_noalloc_scratch_bytes(B, T, C) <= \
            lib.wkv_forward_noalloc_max_scratch()
        x = wkv_inputs.generate("l3b", seed=seed, B=B, T=T, C=C, with_dy=False)
        t = {n: torch.from_numpy(np.ascontiguousarray(x[n])).to(dev) for n in x}
        y = torch.empty_like(t["k"])
        y_ref = torch.empty_like(t["k"])
        args = (B, T, C, _p(t["w"]), _p(t["u"]), _p(t["k"]), _p(t["v"]))
        assert lib.wkv_forward_noalloc(*args, _p(y), st) == wkv.WKV_OK
        assert lib.wkv_forward(*args, _p(y_ref), st) == wkv.WKV_OK
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), "B=%d T=%d C=%d" % (B, T, C)
        ref = oracle.forward_recurrent(x["w"], x["u"], x["k"], x["v"])
        v = assert_wkv_close(y.cpu().numpy(), ref, "noalloc B=%d T=%d C=%d" % (B, T, C))
        print("[noalloc] B=%d T=%d C=%d max_violation=%.3g" % (B, T, C, v), flush=True)


def test_noalloc_refuses_sizes_beyond_its_scratch(wkv, dev):
    lib = wkv.load_library()
    f = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(5)]
    assert lib.wkv_forward_noalloc(16, 4096, 2560, *f, None) == wkv.WKV_ERR_INVALID_ARG
    assert b"scratch" in lib.wkv_last_error()
