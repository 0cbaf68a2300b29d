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


def test_poll_limit_setting(pkg):
    lib = pkg.load_library()
    assert lib.wkv_poll_limit() == 2000
    assert lib.wkv_set_poll_limit(-1) == pkg.WKV_ERR_INVALID_ARG
    assert b"negative" in lib.wkv_last_error()
    assert pkg.set_poll_limit(0) == 2000
    assert lib.wkv_poll_limit() == 0
    assert pkg.set_poll_limit(2000) == 0
    with pytest.raises(pkg.WKVError):
        pkg.set_poll_limit(-5)
    assert lib.wkv_poll_limit() == 2000


def test_status_strings_and_version(pkg):
    lib = pkg.load_library()
    assert lib.wkv_version() >= 100
    assert lib.wkv_status_string(0) == b"ok"
    assert lib.wkv_status_string(1) == b"invalid argument"
    assert lib.wkv_status_string(2) == b"unsupported device"
    assert lib.wkv_status_string(3) == b"HIP runtime error"
    assert lib.wkv_status_string(99) == b"unknown status"


def _r256(x):
    return (x + 255) // 256 * 256


def _fwd_bytes(B, T, C, window=64, chunk=32):
    """Forward workspace: a 256-byte stamp, flags, window aggregates and inclusive carries
    (40 B records), the carry entering each chunk of a window but its first (5 fp64 fields),
    the carry entering token 0 (40 B per sequence and channel) and the final fp32 state
    (12 B)."""
    nseg, ngrp = -(-T // window), -(-C // 64)
    kept = window // chunk - 1
    return (256 + _r256(B * ngrp * nseg * 8) + 2 * _r256(B * nseg * C * 40)
            + _r256(B * nseg * kept * C * 40) + _r256(B * C * 40) + _r256(B * C * 12))


def _bwd_bytes(B, T, C, window=64):
    """Backward workspace: flags, reverse aggregates and inclusive carries (24 B records),
    dw/du partials (2 fp64), and one 24 B record per (b, c) for a final state's cotangent."""
    nseg, ngrp = -(-T // window), -(-C // 64)
    return (_r256(B * ngrp * nseg * 8) + 2 * _r256(B * nseg * C * 24) + _r256(B * nseg * C * 16)
            + _r256(B * C * 24))


def test_sizes(pkg):
    lib = pkg.load_library()
    for B, T, C in ((8, 4096, 2560), (1, 257, 3), (3, 1, 65), (2, 129, 128)):
        fwd = _fwd_bytes(B, T, C)
        assert lib.wkv_forward_workspace_size(B, T, C) == fwd
        own = _bwd_bytes(B, T, C)
        assert lib.wkv_backward_workspace_size_ex(B, T, C, 1) == own
        assert lib.wkv_backward_workspace_size_ex(B, T, C, 0) == own + fwd
        assert lib.wkv_backward_train_workspace_size(B, T, C) == own
        assert lib.wkv_backward_workspace_size(B, T, C) == own + fwd
    assert lib.wkv_forward_workspace_size(1, 257, 3) == 256 + 256 + 2 * 768 + 768 + 256 + 256
    assert lib.wkv_backward_workspace_size(-1, 4, 4) == 0
    assert lib.wkv_forward_workspace_size(-1, 4, 4) == 0
    assert lib.wkv_forward_workspace_size(1, 4, (1 << 24) + 1) == 0


FAKE = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(12)]


def _fwd(lib, B, T, C, ptrs=None, ws=FAKE[6], wsbytes=1 << 40):
    p = FAKE if ptrs is None else ptrs
    return lib.wkv_forward_train(B, T, C, p[0], p[1], p[2], p[3], p[4], ws, wsbytes, None)


def test_plain_forward_signature_and_validation(pkg):
    """wkv_forward(B, T, C, w, u, k, v, y, stream): the same argument checks as the training
    forward, all before any device call (so none of these reaches the GPU)."""
    lib = pkg.load_library()
    f = FAKE

    def call(B=2, T=3, C=4, p=None):
        q = f if p is None else p
        return lib.wkv_forward(B, T, C, q[0], q[1], q[2], q[3], q[4], None)

    assert call(B=-1) == pkg.WKV_ERR_INVALID_ARG
    assert b"negative" in lib.wkv_last_error()
    assert call(C=(1 << 24) + 1) == pkg.WKV_ERR_INVALID_ARG
    assert call(p=[f[0], f[1], None, f[3], f[4]]) == pkg.WKV_ERR_INVALID_ARG
    assert b"k is NULL" in lib.wkv_last_error()
    assert call(p=[f[0], f[1], f[2], f[3], ctypes.c_void_p(f[2].value + 16)]) == \
        pkg.WKV_ERR_INVALID_ARG
    assert b"overlaps" in lib.wkv_last_error()
    assert call(p=[f[0], f[1], f[2], ctypes.c_void_p(0x300002), f[4]]) == pkg.WKV_ERR_INVALID_ARG
    assert b"aligned" in lib.wkv_last_error()
    for B, T, C in ((0, 5, 5), (3, 0, 5), (3, 5, 0)):
        assert call(B, T, C, [None] * 5) == pkg.WKV_OK
    assert lib.wkv_last_error() == b""


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
    assert _fwd(lib, 2, 300, 4, wsbytes=10) == pkg.WKV_ERR_INVALID_ARG
    assert b"workspace has 10 bytes" in lib.wkv_last_error()
    assert _fwd(lib, 2, 300, 4, ws=None) == pkg.WKV_ERR_INVALID_ARG
    assert b"workspace is NULL" in lib.wkv_last_error()
    assert _fwd(lib, 2, 300, 4, ws=ctypes.c_void_p(FAKE[6].value + 8)) == pkg.WKV_ERR_INVALID_ARG
    assert b"16-byte aligned" in lib.wkv_last_error()
    # a workspace overlapping k
    assert _fwd(lib, 2, 300, 4, ws=ctypes.c_void_p(FAKE[2].value + 64)) == pkg.WKV_ERR_INVALID_ARG


def test_forward_state_rejects_bad_arguments(pkg):
    lib = pkg.load_library()
    f = FAKE
    ab, bb, pb = (ctypes.c_void_p(0x900000 + 0x10000 * i) for i in range(3))

    def call(a=ab, b=bb, p=pb, B=2, T=3, C=4):
        return lib.wkv_forward_state(B, T, C, f[0], f[1], f[2], f[3], f[4], a, b, p, f[6],
                                     1 << 40, None)

    assert call(a=None) == pkg.WKV_ERR_INVALID_ARG
    assert b"a is NULL" in lib.wkv_last_error()
    assert call(p=None) == pkg.WKV_ERR_INVALID_ARG
    assert b"p is NULL" in lib.wkv_last_error()
    assert call(b=ctypes.c_void_p(f[2].value + 8)) == pkg.WKV_ERR_INVALID_ARG  # inside k
    assert b"state b overlaps" in lib.wkv_last_error()
    assert call(b=ctypes.c_void_p(ab.value + 4)) == pkg.WKV_ERR_INVALID_ARG
    assert b"state b overlaps state a" in lib.wkv_last_error()
    assert call(a=ctypes.c_void_p(0x900002)) == pkg.WKV_ERR_INVALID_ARG
    assert b"aligned" in lib.wkv_last_error()
    # zero-sized: a no-op that touches nothing, state pointers not needed
    assert call(a=None, b=None, p=None, T=0) == pkg.WKV_OK
    assert lib.wkv_last_error() == b""


def test_typed_entry_points_reject_bad_arguments(pkg):
    lib = pkg.load_library()
    f = FAKE

    def fwd(dtype, k=f[2], r=None):
        return lib.wkv_forward_typed(dtype, 2, 3, 4, f[0], f[1], k, f[3], r, f[4], f[6],
                                     1 << 40, None)

    assert fwd(7) == pkg.WKV_ERR_INVALID_ARG
    assert b"unknown dtype 7" in lib.wkv_last_error()
    # 16-bit tensors need 2-byte alignment only, fp32 ones 4
    assert fwd(pkg.WKV_BF16, k=ctypes.c_void_p(f[2].value + 1)) == pkg.WKV_ERR_INVALID_ARG
    assert b"2-byte aligned" in lib.wkv_last_error()
    assert fwd(pkg.WKV_F32, k=ctypes.c_void_p(f[2].value + 2)) == pkg.WKV_ERR_INVALID_ARG
    assert b"4-byte aligned" in lib.wkv_last_error()

    def bwd(dtype, r=None, dr=None):
        return lib.wkv_backward_typed(dtype, 2, 3, 4, f[0], f[1], f[2], f[3], f[4], r, None,
                                      f[5], f[6], dr, f[9], f[10], f[11], 1 << 40, None)

    assert bwd(pkg.WKV_F16, r=f[7]) == pkg.WKV_ERR_INVALID_ARG
    assert b"r and dr must be given together" in lib.wkv_last_error()
    assert bwd(-1) == pkg.WKV_ERR_INVALID_ARG
    assert b"unknown dtype" in lib.wkv_last_error()


def test_token_shift_rejects_bad_arguments(pkg):
    lib = pkg.load_library()
    f = FAKE
    assert lib.wkv_token_shift(2, 3, 4, None, None, f[1], f[2], f[3], f[4], None,
                               None) == pkg.WKV_ERR_INVALID_ARG
    assert b"x is NULL" in lib.wkv_last_error()
    # an output overlapping x
    assert lib.wkv_token_shift(2, 3, 4, f[0], None, f[1], ctypes.c_void_p(f[0].value + 8), f[3],
                               f[4], None, None) == pkg.WKV_ERR_INVALID_ARG
    assert b"out_r overlaps x" in lib.wkv_last_error()
    assert lib.wkv_token_shift(0, 3, 4, *([None] * 7), None) == pkg.WKV_OK
    # fp64 partials of dmu: 3 fields x B x ceil(T / 32) stretches x C
    assert lib.wkv_token_shift_backward_workspace_size(8, 4096, 2560) == 3 * 8 * 128 * 2560 * 8
    assert lib.wkv_token_shift_backward(2, 3, 4, f[0], None, f[1], f[2], f[3], f[4], f[5], None,
                                        f[6], f[7], 10, None) == pkg.WKV_ERR_INVALID_ARG
    assert b"workspace has 10 bytes" in lib.wkv_last_error()


def test_zero_sized_forward_is_a_noop(pkg):
    lib = pkg.load_library()
    none = [None] * 5
    assert _fwd(lib, 0, 5, 5, none, ws=None) == pkg.WKV_OK
    assert _fwd(lib, 3, 0, 5, none, ws=None) == pkg.WKV_OK
    assert _fwd(lib, 3, 5, 0, none, ws=None) == pkg.WKV_OK
    assert lib.wkv_last_error() == b""


def test_forward_infer_rejects_bad_arguments(pkg):
    lib = pkg.load_library()
    f = FAKE

    def call(dtype=0, a=f[7], b=f[8], p=f[9], B=2, T=3, C=4, ws=f[6]):
        return lib.wkv_forward_infer(dtype, B, T, C, f[0], f[1], f[2], f[3], None, f[4], a, b, p,
                                     ws, 1 << 40, None)

    assert call(dtype=7) == pkg.WKV_ERR_INVALID_ARG
    assert b"unknown dtype" in lib.wkv_last_error()
    assert call(b=None) == pkg.WKV_ERR_INVALID_ARG
    assert b"all of a, b, p or none" in lib.wkv_last_error()
    assert call(ws=None) == pkg.WKV_ERR_INVALID_ARG
    assert call(B=0, ws=None, a=None, b=None, p=None) == pkg.WKV_OK
    # the state overlapping the output
    assert call(a=f[4]) == pkg.WKV_ERR_INVALID_ARG
    assert b"overlaps" in lib.wkv_last_error()


def _bwd(lib, B, T, C, fws=None, ws=FAKE[11], wsbytes=1 << 40, dw=FAKE[9], du=FAKE[10]):
    f = FAKE
    if fws is None:
        return lib.wkv_backward(B, T, C, f[0], f[1], f[2], f[3], f[4], f[5], f[6], dw, du, ws,
                                wsbytes, None)
    return lib.wkv_backward_train(B, T, C, f[0], f[1], f[2], f[3], f[4], fws, f[5], f[6], dw,
                                  du, ws, wsbytes, None)


def test_backward_rejects_bad_arguments(pkg):
    lib = pkg.load_library()
    assert _bwd(lib, 2, -3, 4) == pkg.WKV_ERR_INVALID_ARG
    assert _bwd(lib, 2, 3, 4, dw=None) == pkg.WKV_ERR_INVALID_ARG
    assert b"dw is NULL" in lib.wkv_last_error()
    assert _bwd(lib, 2, 3, 4, ws=None) == pkg.WKV_ERR_INVALID_ARG
    assert b"workspace is NULL" in lib.wkv_last_error()
    assert _bwd(lib, 2, 3, 4, wsbytes=100) == pkg.WKV_ERR_INVALID_ARG
    assert b"workspace has 100 bytes" in lib.wkv_last_error()
    # dk aliasing dy
    f = FAKE
    rc = lib.wkv_backward(2, 3, 4, f[0], f[1], f[2], f[3], f[4], f[4], f[6], f[9], f[10],
                          f[11], 1 << 40, None)
    assert rc == pkg.WKV_ERR_INVALID_ARG and b"overlaps" in lib.wkv_last_error()
    assert _bwd(lib, 2, 3, 0, dw=None, du=None) == pkg.WKV_OK
    # the training backward: its forward workspace is required, and its own workspace is the
    # smaller one
    rc = lib.wkv_backward_train(2, 3, 4, f[0], f[1], f[2], f[3], f[4], None, f[5], f[6], f[9],
                                f[10], f[11], 1 << 40, None)
    assert rc == pkg.WKV_ERR_INVALID_ARG and b"fwd_workspace is NULL" in lib.wkv_last_error()
    need = lib.wkv_backward_train_workspace_size(2, 300, 4)
    assert _bwd(lib, 2, 300, 4, fws=f[7], wsbytes=need - 1) == pkg.WKV_ERR_INVALID_ARG
    assert b"workspace has" in lib.wkv_last_error()


def test_backward_state_rejects_bad_arguments(pkg):
    # every call here fails validation (or has nothing to do) before any device call
    lib = pkg.load_library()
    g = [ctypes.c_void_p(0x4000000 + 0x100000 * i) for i in range(16)]

    def call(B=2, T=3, C=4, fws=g[5], da=g[12], db=g[13], dp=g[14], dfa=None, dfb=None):
        return lib.wkv_backward_state(B, T, C, g[0], g[1], g[2], g[3], g[4], dfa, dfb, fws,
                                      g[6], g[7], g[8], g[9], da, db, dp, g[11], 1 << 40, None)

    assert call(T=-1) == pkg.WKV_ERR_INVALID_ARG
    assert call(fws=None) == pkg.WKV_ERR_INVALID_ARG
    assert b"fwd_workspace is NULL" in lib.wkv_last_error()
    assert call(T=0, fws=None) == pkg.WKV_ERR_INVALID_ARG
    assert call(db=None) == pkg.WKV_ERR_INVALID_ARG
    assert b"db is NULL" in lib.wkv_last_error()
    assert call(dp=ctypes.c_void_p(g[14].value + 2)) == pkg.WKV_ERR_INVALID_ARG
    assert call(db=ctypes.c_void_p(g[12].value + 16)) == pkg.WKV_ERR_INVALID_ARG
    assert b"overlap" in lib.wkv_last_error()
    # da on top of an input (k) and of another output (dk)
    assert call(da=g[2]) == pkg.WKV_ERR_INVALID_ARG
    assert b"overlaps an input" in lib.wkv_last_error()
    assert call(dp=g[6]) == pkg.WKV_ERR_INVALID_ARG
    assert b"two outputs overlap" in lib.wkv_last_error()
    # the final state's cotangent: both or neither, not for T = 0, not on an output
    assert call(dfa=g[10]) == pkg.WKV_ERR_INVALID_ARG
    assert b"both of dfa, dfb" in lib.wkv_last_error()
    assert call(T=0, dfa=g[10], dfb=g[15]) == pkg.WKV_ERR_INVALID_ARG
    assert b"T = 0" in lib.wkv_last_error()
    assert call(dfa=g[10], dfb=ctypes.c_void_p(g[15].value + 1)) == pkg.WKV_ERR_INVALID_ARG
    assert call(dfa=g[10], dfb=g[13]) == pkg.WKV_ERR_INVALID_ARG
    assert b"overlaps an input" in lib.wkv_last_error()
    assert lib.wkv_backward_state(2, 3, 0, *([None] * 16), 0, None) == pkg.WKV_OK
    # the typed form: unknown dtype, r without dr, and the same checks as above
    assert lib.wkv_backward_state_typed(7, 2, 3, 4, *g[:5], None, None, None, g[5], g[6],
                                        g[7], None, g[8], g[9], g[12], g[13], g[14], g[11],
                                        1 << 40, None) == pkg.WKV_ERR_INVALID_ARG
    assert b"unknown dtype" in lib.wkv_last_error()
    assert lib.wkv_backward_state_typed(1, 2, 3, 4, *g[:5], g[15], None, None, g[5], g[6],
                                        g[7], None, g[8], g[9], g[12], g[13], g[14], g[11],
                                        1 << 40, None) == pkg.WKV_ERR_INVALID_ARG
    assert b"r and dr" in lib.wkv_last_error()
    assert lib.wkv_backward_state_typed(1, 2, 3, 4, *g[:5], None, None, None, None, g[6],
                                        g[7], None, g[8], g[9], g[12], g[13], g[14], g[11],
                                        1 << 40, None) == pkg.WKV_ERR_INVALID_ARG
    assert b"fwd_workspace is NULL" in lib.wkv_last_error()
    assert lib.wkv_forward_state_typed(5, 2, 3, 4, *g[:4], None, g[4], g[12], g[13], g[14],
                                       g[11], 1 << 40, None) == pkg.WKV_ERR_INVALID_ARG
    assert lib.wkv_forward_state_typed(1, 2, 3, 4, *g[:4], None, g[4], g[12], None, g[14],
                                       g[11], 1 << 40, None) == pkg.WKV_ERR_INVALID_ARG
    assert b"all of a, b, p or none" in lib.wkv_last_error()


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
    # the 16-bit form: unknown dtype, 2-byte alignment of k, v, y, 4-byte of the state
    assert lib.wkv_decode_step_typed(9, 2, 3, *f[:8], None) == pkg.WKV_ERR_INVALID_ARG
    assert b"unknown dtype" in lib.wkv_last_error()
    odd = ctypes.c_void_p(f[2].value + 1)
    assert lib.wkv_decode_step_typed(1, 2, 3, f[0], f[1], odd, f[3], f[4], f[5], f[6], f[7],
                                     None) == pkg.WKV_ERR_INVALID_ARG
    half = ctypes.c_void_p(f[4].value + 2)
    assert lib.wkv_decode_step_typed(1, 2, 3, f[0], f[1], f[2], f[3], half, f[5], f[6], f[7],
                                     None) == pkg.WKV_ERR_INVALID_ARG
    assert lib.wkv_decode_step_typed(1, 2, 3, f[0], f[1], f[2], f[3], f[4], f[5], f[6], f[4],
                                     None) == pkg.WKV_ERR_INVALID_ARG
    assert b"overlaps" in lib.wkv_last_error()
    assert lib.wkv_decode_step_typed(2, 0, 3, *([None] * 8), None) == pkg.WKV_OK


def test_python_layer_rejects_bad_tensors(pkg):
    import torch
    x = torch.zeros(2, 3, 4)
    with pytest.raises(ValueError):
        pkg.forward(torch.zeros(4), torch.zeros(4), x, x)  # CPU tensors
    with pytest.raises(TypeError):
        pkg.forward(torch.zeros(4), torch.zeros(4), x.double(), x)


def test_missing_library_fails_loudly_with_its_path(tmp_path):
    """No CPU fallback: a library that is not there is an ImportError naming the path
    (RWKV_WKV_LIB points the binding at a copy; here at a file that does not exist)."""
    import subprocess
    import sys
    missing = str(tmp_path / "no_such_librwkv_wkv.so")
    env = dict(os.environ, RWKV_WKV_LIB=missing)
    code = ("import sys; sys.path.insert(0, %r)\n"
            "try:\n"
            "    import rwkv_linear_attention_forward_amd\n"
            "except ImportError as e:\n"
            "    print('IMPORTERROR', e)\n" % os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "IMPORTERROR" in r.stdout and missing in r.stdout
