"""The C-ABI library loads, exports every declared symbol, and validates arguments on
the host before any HIP call (CPU only: no kernel is launched here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rwkv_wkv.h")


@pytest.fixture(scope="module")
def pkg():
    import rwkv_linear_attention_forward_amd as m
    return m


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\w[\w\s\*]*?\b(wkv_\w+)\s*\(", src, re.M)))


def test_header_declarations_match_binding(pkg):
    assert _declared() == sorted(pkg.EXPORTS)


def test_every_declared_symbol_is_exported(pkg):
    lib = ctypes.CDLL(pkg.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name


def test_status_strings_and_version(pkg):
    lib = pkg.load_library()
    assert lib.wkv_version() >= 100
    assert lib.wkv_status_string(0) == b"ok"
    assert lib.wkv_status_string(1) == b"invalid argument"
    assert lib.wkv_status_string(2) == b"unsupported device"
    assert lib.wkv_status_string(3) == b"HIP runtime error"
    assert lib.wkv_status_string(99) == b"unknown status"


def test_sizes(pkg):
    lib = pkg.load_library()
    assert lib.wkv_saved_size(8, 4096, 2560) == 8 * 16 * 2560 * 16
    assert lib.wkv_saved_size(1, 257, 3) == 1 * 2 * 3 * 16
    assert lib.wkv_saved_size(-1, 4, 4) == 0
    assert lib.wkv_saved_size(1, 4, (1 << 24) + 1) == 0
    assert lib.wkv_backward_workspace_size(8, 4096, 2560, 1) == 8 * 2560 * 16
    assert (lib.wkv_backward_workspace_size(8, 4096, 2560, 0)
            == 8 * 2560 * 16 + 8 * 16 * 2560 * 16)
    assert lib.wkv_backward_workspace_size(1, 1, 3, 1) == 256  # rounded to 256 bytes


FAKE = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(12)]


def _fwd(lib, B, T, C, ptrs=None, saved=None, sbytes=0):
    p = FAKE if ptrs is None else ptrs
    return lib.wkv_forward(B, T, C, p[0], p[1], p[2], p[3], p[4], saved, sbytes, None)


def test_forward_rejects_bad_arguments(pkg):
    lib = pkg.load_library()
    assert _fwd(lib, -1, 4, 4) == pkg.WKV_ERR_INVALID_ARG
    assert b"negative" in lib.wkv_last_error()
    assert _fwd(lib, 1, 4, (1 << 24) + 1) == pkg.WKV_ERR_INVALID_ARG
    assert _fwd(lib, 1 << 40, 1 << 20, 64) == pkg.WKV_ERR_INVALID_ARG
    assert b"overflow" in lib.wkv_last_error()
    nul = [FAKE[0], FAKE[1], None, FAKE[3], FAKE[4]]
    assert _fwd(lib, 2, 3, 4, nul) == pkg.WKV_ERR_INVALID_ARG
    assert b"k is NULL" in lib.wkv_last_error()
    odd = [FAKE[0], FAKE[1], FAKE[2], ctypes.c_void_p(0x300002), FAKE[4]]
    assert _fwd(lib, 2, 3, 4, odd) == pkg.WKV_ERR_INVALID_ARG
    assert b"aligned" in lib.wkv_last_error()
    alias = [FAKE[0], FAKE[1], FAKE[2], FAKE[3], ctypes.c_void_p(FAKE[2].value + 16)]
    assert _fwd(lib, 2, 3, 4, alias) == pkg.WKV_ERR_INVALID_ARG
    assert b"overlaps" in lib.wkv_last_error()
    assert _fwd(lib, 2, 300, 4, saved=FAKE[6], sbytes=10) == pkg.WKV_ERR_INVALID_ARG
    assert b"saved buffer" in lib.wkv_last_error()


def test_zero_sized_forward_is_a_noop(pkg):
    lib = pkg.load_library()
    none = [None] * 5
    assert _fwd(lib, 0, 5, 5, none) == pkg.WKV_OK
    assert _fwd(lib, 3, 0, 5, none) == pkg.WKV_OK
    assert _fwd(lib, 3, 5, 0, none) == pkg.WKV_OK
    assert lib.wkv_last_error() == b""


def test_decode_rejects_bad_arguments(pkg):
    lib = pkg.load_library()
    f = FAKE
    assert lib.wkv_decode_step(-2, 3, *f[:8], None) == pkg.WKV_ERR_INVALID_ARG
    assert lib.wkv_decode_step(2, 3, f[0], f[1], f[2], f[3], None, f[5], f[6], f[7],
                               None) == pkg.WKV_ERR_INVALID_ARG
    assert b"a is NULL" in lib.wkv_last_error()
    # y aliasing the state
    assert lib.wkv_decode_step(2, 3, f[0], f[1], f[2], f[3], f[4], f[5], f[6], f[4],
                               None) == pkg.WKV_ERR_INVALID_ARG
    assert b"overlaps" in lib.wkv_last_error()
    assert lib.wkv_decode_step(0, 3, *([None] * 8), None) == pkg.WKV_OK


def test_python_layer_rejects_bad_tensors(pkg):
    import torch
    x = torch.zeros(2, 3, 4)
    with pytest.raises(ValueError):
        pkg.forward(torch.zeros(4), torch.zeros(4), x, x)  # CPU tensors
    with pytest.raises(TypeError):
        pkg.forward(torch.zeros(4), torch.zeros(4), x.double(), x)
