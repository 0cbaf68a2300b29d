"""Python binding of librwkv_wkv, the RWKV-4 WKV operator for MI355X (gfx950).

Argument marshalling only: every step of the operator runs in the HIP kernels of
librwkv_wkv.so (built in-tree by ``build.py``); PyTorch provides device memory and the
current stream. Importing this module loads the library (or the file RWKV_WKV_LIB names) and fails
loudly, with an ImportError naming the path, if it is not there; there is no CPU fallback.

Entry points mirror the C ABI in include/rwkv_wkv.h:

    forward(w, u, k, v, workspace=None) -> y      (with a workspace: the training forward)
    forward_state(w, u, k, v, a, b, p, workspace=None) -> y   (a, b, p: state in, state out)
    forward_gated(w, u, k, v, r, workspace=None) -> sigma(r) * y
    backward_gated(w, u, k, v, r, dout, fwd_workspace=None) -> (dk, dv, dr, dw, du)
    forward_workspace(B, T, C, device) -> uint8 tensor sized for the forward
    backward(w, u, k, v, dy, fwd_workspace=None) -> (dk, dv, dw, du)
                                    (with fwd_workspace: the training backward)
    decode_step(w, u, k, v, a, b, p) -> y          (a, b, p updated in place)
    token_shift(x, mu, x_prev=None) -> (out_r, out_k, out_v, x_last)
    token_shift_backward(x, mu, dout, x_prev=None) -> (dx, dx_prev, dmu)

Operator ("RWKV解读：在Transformer的时代的新RNN", section 二.3, formula (8)):
    y_t = (sum_{i<t} e^{-(t-1-i)w + k_i} v_i + e^{u+k_t} v_t)
        / (sum_{i<t} e^{-(t-1-i)w + k_i}     + e^{u+k_t})
"""
from __future__ import annotations

import ctypes
import os

import torch  # first: its HIP runtime is the one the library binds to

_PKG = os.path.dirname(os.path.abspath(__file__))
# the in-tree build, unless RWKV_WKV_LIB names another copy of the library
LIB_PATH = os.environ.get("RWKV_WKV_LIB") or os.path.join(_PKG, "librwkv_wkv.so")

WKV_OK = 0
WKV_ERR_INVALID_ARG = 1
WKV_ERR_UNSUPPORTED = 2
WKV_ERR_HIP = 3

# Every symbol the header declares, for the export check.
EXPORTS = ("wkv_version", "wkv_set_poll_limit", "wkv_poll_limit", "wkv_status_string",
           "wkv_last_error", "wkv_forward_workspace_size",
           "wkv_forward", "wkv_forward_noalloc", "wkv_forward_noalloc_scratch_bytes",
           "wkv_forward_noalloc_max_scratch",
           "wkv_forward_train", "wkv_forward_state", "wkv_forward_gated",
           "wkv_forward_typed", "wkv_forward_infer",
           "wkv_backward_workspace_size", "wkv_backward_train_workspace_size",
           "wkv_backward_workspace_size_ex", "wkv_backward", "wkv_backward_train",
           "wkv_backward_gated",
           "wkv_backward_typed", "wkv_backward_state", "wkv_forward_state_typed",
           "wkv_backward_state_typed", "wkv_decode_step",
           "wkv_decode_step_typed", "wkv_token_shift",
           "wkv_token_shift_backward_workspace_size", "wkv_token_shift_backward")

# Storage formats of the [B, T, C] tensors (dtype codes of the *_typed entry points).
WKV_F32, WKV_BF16, WKV_F16 = 0, 1, 2
_DTYPE_CODE = {torch.float32: WKV_F32, torch.bfloat16: WKV_BF16, torch.float16: WKV_F16}

_lib = None
_I64 = ctypes.c_int64
_P = ctypes.c_void_p


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load (once) and type the C ABI. Raises ImportError if the library is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError("librwkv_wkv.so not found at %s: run "
                          "`python rwkv_linear_attention_forward_amd/build.py`" % path)
    lib = ctypes.CDLL(path)
    lib.wkv_version.restype = ctypes.c_int
    lib.wkv_version.argtypes = []
    lib.wkv_set_poll_limit.restype = ctypes.c_int
    lib.wkv_set_poll_limit.argtypes = [ctypes.c_int]
    lib.wkv_poll_limit.restype = ctypes.c_int
    lib.wkv_poll_limit.argtypes = []
    lib.wkv_status_string.restype = ctypes.c_char_p
    lib.wkv_status_string.argtypes = [ctypes.c_int]
    lib.wkv_last_error.restype = ctypes.c_char_p
    lib.wkv_last_error.argtypes = []
    lib.wkv_forward_workspace_size.restype = ctypes.c_size_t
    lib.wkv_forward_workspace_size.argtypes = [_I64, _I64, _I64]
    lib.wkv_forward.restype = ctypes.c_int
    lib.wkv_forward.argtypes = [_I64, _I64, _I64, _P, _P, _P, _P, _P, _P]
    lib.wkv_forward_noalloc.restype = ctypes.c_int
    lib.wkv_forward_noalloc.argtypes = [_I64, _I64, _I64, _P, _P, _P, _P, _P, _P]
    lib.wkv_forward_noalloc_scratch_bytes.restype = ctypes.c_size_t
    lib.wkv_forward_noalloc_scratch_bytes.argtypes = [_I64, _I64, _I64]
    lib.wkv_forward_noalloc_max_scratch.restype = ctypes.c_size_t
    lib.wkv_forward_noalloc_max_scratch.argtypes = []
    lib.wkv_forward_train.restype = ctypes.c_int
    lib.wkv_forward_train.argtypes = [_I64, _I64, _I64, _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                                      _P]
    lib.wkv_forward_typed.restype = ctypes.c_int
    lib.wkv_forward_typed.argtypes = [ctypes.c_int, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P,
                                      ctypes.c_size_t, _P]
    lib.wkv_forward_infer.restype = ctypes.c_int
    lib.wkv_forward_infer.argtypes = [ctypes.c_int, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P,
                                      _P, _P, _P, ctypes.c_size_t, _P]
    lib.wkv_backward_typed.restype = ctypes.c_int
    lib.wkv_backward_typed.argtypes = [ctypes.c_int, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P,
                                       _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.wkv_token_shift.restype = ctypes.c_int
    lib.wkv_token_shift.argtypes = [_I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.wkv_token_shift_backward_workspace_size.restype = ctypes.c_size_t
    lib.wkv_token_shift_backward_workspace_size.argtypes = [_I64, _I64, _I64]
    lib.wkv_token_shift_backward.restype = ctypes.c_int
    lib.wkv_token_shift_backward.argtypes = [_I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                             _P, ctypes.c_size_t, _P]
    lib.wkv_forward_gated.restype = ctypes.c_int
    lib.wkv_forward_gated.argtypes = [_I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P,
                                      ctypes.c_size_t, _P]
    lib.wkv_backward_gated.restype = ctypes.c_int
    lib.wkv_backward_gated.argtypes = [_I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                       _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.wkv_forward_state.restype = ctypes.c_int
    lib.wkv_forward_state.argtypes = [_I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                      ctypes.c_size_t, _P]
    for name in ("wkv_backward_workspace_size", "wkv_backward_train_workspace_size"):
        getattr(lib, name).restype = ctypes.c_size_t
        getattr(lib, name).argtypes = [_I64, _I64, _I64]
    lib.wkv_backward_workspace_size_ex.restype = ctypes.c_size_t
    lib.wkv_backward_workspace_size_ex.argtypes = [_I64, _I64, _I64, ctypes.c_int]
    lib.wkv_backward.restype = ctypes.c_int
    lib.wkv_backward.argtypes = [_I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                 ctypes.c_size_t, _P]
    lib.wkv_backward_train.restype = ctypes.c_int
    lib.wkv_backward_train.argtypes = [_I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                       _P, ctypes.c_size_t, _P]
    lib.wkv_backward_state.restype = ctypes.c_int
    lib.wkv_backward_state.argtypes = [_I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                       _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.wkv_forward_state_typed.restype = ctypes.c_int
    lib.wkv_forward_state_typed.argtypes = [ctypes.c_int, _I64, _I64, _I64, _P, _P, _P, _P, _P,
                                            _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.wkv_backward_state_typed.restype = ctypes.c_int
    lib.wkv_backward_state_typed.argtypes = [ctypes.c_int, _I64, _I64, _I64, _P, _P, _P, _P, _P,
                                             _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                             ctypes.c_size_t, _P]
    lib.wkv_decode_step_typed.restype = ctypes.c_int
    lib.wkv_decode_step_typed.argtypes = [ctypes.c_int, _I64, _I64, _P, _P, _P, _P, _P, _P, _P,
                                          _P, _P]
    lib.wkv_decode_step.restype = ctypes.c_int
    lib.wkv_decode_step.argtypes = [_I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P]
    _lib = lib
    return lib


class WKVError(RuntimeError):
    """A nonzero status from librwkv_wkv, with the library's message."""

    def __init__(self, status: int, message: str):
        super().__init__("%s (status %d): %s" % (_status_name(status), status, message))
        self.status = status


def _status_name(status: int) -> str:
    return load_library().wkv_status_string(status).decode()


def _check(status: int):
    if status != WKV_OK:
        raise WKVError(status, load_library().wkv_last_error().decode())


def set_poll_limit(tries: int) -> int:
    """Set how many times a look-back re-reads an unpublished window's flag before it
    recomputes that window itself (results are bitwise the same either way); returns the
    previous setting."""
    lib = load_library()
    old = lib.wkv_poll_limit()
    _check(lib.wkv_set_poll_limit(int(tries)))
    return old


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, ndim, device=None, dtype=torch.float32):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_cuda:
        raise ValueError("%s must be on a GPU device" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if t.dim() != ndim:
        raise ValueError("%s must have %d dims, got shape %s" % (name, ndim, tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _check_btc(w, u, k, v, typed=False):
    """Shapes and devices of the operands. With typed=True the [B, T, C] tensors may be
    float32, bfloat16 or float16 (all the same); w and u are always float32."""
    if not isinstance(k, torch.Tensor):
        raise TypeError("k must be a torch.Tensor")
    if typed and k.dtype not in _DTYPE_CODE:
        raise TypeError("k must be float32, bfloat16 or float16, got %s" % k.dtype)
    _need(k, "k", 3, dtype=k.dtype if typed else torch.float32)
    dev = k.device
    _need(v, "v", 3, dev, dtype=k.dtype)
    _need(w, "w", 1, dev)
    _need(u, "u", 1, dev)
    B, T, C = k.shape
    if v.shape != k.shape:
        raise ValueError("v shape %s != k shape %s" % (tuple(v.shape), tuple(k.shape)))
    if w.shape[0] != C or u.shape[0] != C:
        raise ValueError("w and u must have C=%d elements" % C)
    return B, T, C, dev


def forward_workspace_size(B: int, T: int, C: int) -> int:
    """Bytes of scratch wkv_forward needs (it also keeps the states wkv_backward reuses)."""
    return int(load_library().wkv_forward_workspace_size(B, T, C))


def forward_workspace(B: int, T: int, C: int, device) -> torch.Tensor:
    """A uint8 device tensor sized for wkv_forward."""
    return torch.empty(max(16, forward_workspace_size(B, T, C)), dtype=torch.uint8,
                       device=device)


def _check_ws(ws, dev, name):
    if ws.dtype != torch.uint8 or ws.device != dev or not ws.is_contiguous():
        raise ValueError("%s must be a contiguous uint8 tensor on %s" % (name, dev))


def _forward_common(w, u, k, v, r, workspace, out):
    B, T, C, dev = _check_btc(w, u, k, v, typed=True)
    if r is not None:
        _need(r, "r", 3, dev, dtype=k.dtype)
        if r.shape != k.shape:
            raise ValueError("r has the wrong shape")
    y = torch.empty_like(k) if out is None else out
    _need(y, "out", 3, dev, dtype=k.dtype)
    if y.shape != k.shape:
        raise ValueError("out has the wrong shape")
    lib = load_library()
    if workspace is None and r is None and k.dtype == torch.float32:
        # the plain forward: no workspace, nothing kept for a backward
        _check(lib.wkv_forward(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(y),
                               _stream(dev)))
        return y
    if workspace is None:
        workspace = forward_workspace(B, T, C, dev)
    _check_ws(workspace, dev, "workspace")
    if k.dtype == torch.float32:
        if r is None:
            rc = lib.wkv_forward_train(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(y),
                                       _ptr(workspace), workspace.numel(), _stream(dev))
        else:
            rc = lib.wkv_forward_gated(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(r),
                                       _ptr(y), _ptr(workspace), workspace.numel(), _stream(dev))
    else:
        rc = lib.wkv_forward_typed(_DTYPE_CODE[k.dtype], B, T, C, _ptr(w), _ptr(u), _ptr(k),
                                   _ptr(v), _ptr(r), _ptr(y), _ptr(workspace), workspace.numel(),
                                   _stream(dev))
    _check(rc)
    return y


def forward(w, u, k, v, workspace=None, out=None):
    """y [B,T,C] = WKV(w, u, k, v). k, v (and y) are float32, bfloat16 or float16 (all the
    same; w, u float32). With `workspace` (uint8, forward_workspace_size bytes) this is the
    training forward (wkv_forward_train, or wkv_forward_typed for 16-bit storage), which
    leaves in it the states backward() can reuse; without it, float32 inputs go through
    wkv_forward (no workspace, nothing kept) and 16-bit ones through wkv_forward_typed with a
    workspace allocated here."""
    return _forward_common(w, u, k, v, None, workspace, out)


def forward_state(w, u, k, v, a, b, p, workspace=None, out=None, r=None):
    """y [B,T,C] = WKV(w, u, k, v) started from the state (a, b, p) [B,C] float32 (the decode
    convention), which is overwritten with the state after the last token; with r, the
    gated output sigma(r) * y. k, v, r, out share one of float32, bfloat16, float16. The
    workspace keeps what backward_state() reads."""
    B, T, C, dev = _check_btc(w, u, k, v, typed=True)
    for t, n in ((a, "a"), (b, "b"), (p, "p")):
        _need(t, n, 2, dev)
        if tuple(t.shape) != (B, C):
            raise ValueError("%s must have shape %s, got %s" % (n, (B, C), tuple(t.shape)))
    if r is not None:
        _need(r, "r", 3, dev, dtype=k.dtype)
        if r.shape != k.shape:
            raise ValueError("r has the wrong shape")
    y = torch.empty_like(k) if out is None else out
    _need(y, "out", 3, dev, dtype=k.dtype)
    if y.shape != k.shape:
        raise ValueError("out has the wrong shape")
    if workspace is None:
        workspace = forward_workspace(B, T, C, dev)
    _check_ws(workspace, dev, "workspace")
    lib = load_library()
    if k.dtype == torch.float32 and r is None:
        rc = lib.wkv_forward_state(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(y), _ptr(a),
                                   _ptr(b), _ptr(p), _ptr(workspace), workspace.numel(),
                                   _stream(dev))
    else:
        rc = lib.wkv_forward_state_typed(_DTYPE_CODE[k.dtype], B, T, C, _ptr(w), _ptr(u),
                                         _ptr(k), _ptr(v), _ptr(r), _ptr(y), _ptr(a), _ptr(b),
                                         _ptr(p), _ptr(workspace), workspace.numel(),
                                         _stream(dev))
    _check(rc)
    return y


def backward_workspace_size(B: int, T: int, C: int, have_fwd_workspace: bool) -> int:
    """Bytes of the backward's workspace, with or without a forward workspace to read."""
    return int(load_library().wkv_backward_workspace_size_ex(B, T, C,
                                                             1 if have_fwd_workspace else 0))


def _backward_common(w, u, k, v, dy, r, fwd_workspace, workspace, out):
    B, T, C, dev = _check_btc(w, u, k, v, typed=True)
    gated = r is not None
    for t, n in ((dy, "dout" if gated else "dy"),) + (((r, "r"),) if gated else ()):
        _need(t, n, 3, dev, dtype=k.dtype)
        if t.shape != k.shape:
            raise ValueError("%s has the wrong shape" % n)
    if fwd_workspace is not None:
        _check_ws(fwd_workspace, dev, "fwd_workspace")
    wsz = backward_workspace_size(B, T, C, fwd_workspace is not None)
    if workspace is None or workspace.numel() < wsz:
        workspace = torch.empty(max(16, wsz), dtype=torch.uint8, device=dev)
    _check_ws(workspace, dev, "workspace")
    names = ("dk", "dv") + (("dr",) if gated else ()) + ("dw", "du")
    refs = (k, k) + ((k,) if gated else ()) + (w, u)
    if out is None:
        grads = tuple(torch.empty_like(ref) for ref in refs)
    else:
        grads = tuple(out)
        if len(grads) != len(names):
            raise ValueError("out must hold %d tensors" % len(names))
        for t, n, ref in zip(grads, names, refs):
            _need(t, n, ref.dim(), dev, dtype=ref.dtype)
            if t.shape != ref.shape:
                raise ValueError("%s has the wrong shape" % n)
    dk, dv = grads[0], grads[1]
    dr = grads[2] if gated else None
    dw, du = grads[-2], grads[-1]
    lib = load_library()
    if k.dtype == torch.float32 and not gated and fwd_workspace is None:
        rc = lib.wkv_backward(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(dy), _ptr(dk),
                              _ptr(dv), _ptr(dw), _ptr(du), _ptr(workspace), workspace.numel(),
                              _stream(dev))
    elif k.dtype == torch.float32 and not gated:
        rc = lib.wkv_backward_train(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(dy),
                                    _ptr(fwd_workspace), _ptr(dk), _ptr(dv), _ptr(dw), _ptr(du),
                                    _ptr(workspace), workspace.numel(), _stream(dev))
    elif k.dtype == torch.float32:
        rc = lib.wkv_backward_gated(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(r),
                                    _ptr(dy), _ptr(fwd_workspace), _ptr(dk), _ptr(dv), _ptr(dr),
                                    _ptr(dw), _ptr(du), _ptr(workspace), workspace.numel(),
                                    _stream(dev))
    else:
        rc = lib.wkv_backward_typed(_DTYPE_CODE[k.dtype], B, T, C, _ptr(w), _ptr(u), _ptr(k),
                                    _ptr(v), _ptr(dy), _ptr(r), _ptr(fwd_workspace), _ptr(dk),
                                    _ptr(dv), _ptr(dr), _ptr(dw), _ptr(du), _ptr(workspace),
                                    workspace.numel(), _stream(dev))
    _check(rc)
    return grads


def backward(w, u, k, v, dy, fwd_workspace=None, workspace=None, out=None):
    """(dk, dv, dw, du) of sum(dy * y). `fwd_workspace` is the workspace forward() filled for
    the same inputs (optional: without it the window states are recomputed). `out` may hold
    preallocated (dk, dv, dw, du). k, v, dy (and dk, dv) share one of float32, bfloat16,
    float16; w, u, dw, du are float32."""
    return _backward_common(w, u, k, v, dy, None, fwd_workspace, workspace, out)


def backward_state(w, u, k, v, dy, fwd_workspace, dstate=None, workspace=None, out=None,
                   r=None):
    """(dk, dv, dw, du, da, db, dp) for a forward_state() call, whose workspace
    `fwd_workspace` is required: the gradients of sum(dy * y) plus, with `dstate` = (da_T,
    db_T) [B, C], of sum(da_T * a_T + db_T * b_T) for the final state (a_T, b_T, p_T) that
    call returned (the next piece's da, db). da, db, dp [B, C] are the gradient with
    respect to the state (a, b, p) the forward started from (it records both states, so the
    caller need not keep them). With r (a gated forward_state), dy is the cotangent of
    sigma(r) * y and dr follows dv: (dk, dv, dr, dw, du, da, db, dp). k, v, dy, r and dk,
    dv, dr share one of float32, bfloat16, float16; the rest is float32. `out` may hold the
    outputs preallocated."""
    B, T, C, dev = _check_btc(w, u, k, v, typed=True)
    gated = r is not None
    for t, n in ((dy, "dy"),) + (((r, "r"),) if gated else ()):
        _need(t, n, 3, dev, dtype=k.dtype)
        if t.shape != k.shape:
            raise ValueError("%s has the wrong shape" % n)
    if fwd_workspace is None:
        raise ValueError("backward_state needs the workspace of the forward_state call")
    _check_ws(fwd_workspace, dev, "fwd_workspace")
    dfa = dfb = None
    if dstate is not None:
        dfa, dfb = tuple(dstate)
        for t, n in ((dfa, "da_T"), (dfb, "db_T")):
            _need(t, n, 2, dev)
            if tuple(t.shape) != (B, C):
                raise ValueError("%s must have shape %s, got %s" % (n, (B, C), tuple(t.shape)))
    wsz = backward_workspace_size(B, T, C, True)
    if workspace is None or workspace.numel() < wsz:
        workspace = torch.empty(max(16, wsz), dtype=torch.uint8, device=dev)
    _check_ws(workspace, dev, "workspace")
    big = (B, T, C)
    names = ("dk", "dv") + (("dr",) if gated else ()) + ("dw", "du", "da", "db", "dp")
    shapes = (big, big) + ((big,) if gated else ()) + ((C,), (C,), (B, C), (B, C), (B, C))
    dts = (k.dtype, k.dtype) + ((k.dtype,) if gated else ()) + (torch.float32,) * 5
    if out is None:
        grads = tuple(torch.empty(sh, dtype=dt, device=dev) for sh, dt in zip(shapes, dts))
    else:
        grads = tuple(out)
        if len(grads) != len(names):
            raise ValueError("out must hold %d tensors" % len(names))
        for t, n, sh, dt in zip(grads, names, shapes, dts):
            _need(t, n, len(sh), dev, dtype=dt)
            if tuple(t.shape) != sh:
                raise ValueError("%s has the wrong shape" % n)
    dk, dv = grads[0], grads[1]
    dr = grads[2] if gated else None
    dw, du, da, db, dp = grads[-5:]
    lib = load_library()
    if k.dtype == torch.float32 and not gated:
        rc = lib.wkv_backward_state(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(dy),
                                    _ptr(dfa), _ptr(dfb), _ptr(fwd_workspace), _ptr(dk),
                                    _ptr(dv), _ptr(dw), _ptr(du), _ptr(da), _ptr(db), _ptr(dp),
                                    _ptr(workspace), workspace.numel(), _stream(dev))
    else:
        rc = lib.wkv_backward_state_typed(_DTYPE_CODE[k.dtype], B, T, C, _ptr(w), _ptr(u),
                                          _ptr(k), _ptr(v), _ptr(dy), _ptr(r), _ptr(dfa),
                                          _ptr(dfb), _ptr(fwd_workspace), _ptr(dk), _ptr(dv),
                                          _ptr(dr), _ptr(dw), _ptr(du), _ptr(da), _ptr(db),
                                          _ptr(dp), _ptr(workspace), workspace.numel(),
                                          _stream(dev))
    _check(rc)
    return grads


def forward_infer(w, u, k, v, r=None, state=None, workspace=None, out=None):
    """The forward for inference (no backward follows): y, or sigma(r) * y with r, from the
    empty state or from `state` = (a, b, p) [B, C] float32, which is overwritten with the
    state after the last token. k, v, r, out share one of float32, bfloat16, float16. The
    results equal forward() / forward_gated() / forward_state(); the workspace keeps no
    states for backward()."""
    B, T, C, dev = _check_btc(w, u, k, v, typed=True)
    if r is not None:
        _need(r, "r", 3, dev, dtype=k.dtype)
        if r.shape != k.shape:
            raise ValueError("r has the wrong shape")
    st = (None, None, None)
    if state is not None:
        st = tuple(state)
        if len(st) != 3:
            raise ValueError("state must be (a, b, p)")
        for t, n in zip(st, ("a", "b", "p")):
            _need(t, n, 2, dev)
            if tuple(t.shape) != (B, C):
                raise ValueError("%s must have shape %s, got %s" % (n, (B, C), tuple(t.shape)))
    y = torch.empty_like(k) if out is None else out
    _need(y, "out", 3, dev, dtype=k.dtype)
    if y.shape != k.shape:
        raise ValueError("out has the wrong shape")
    if workspace is None:
        workspace = forward_workspace(B, T, C, dev)
    _check_ws(workspace, dev, "workspace")
    _check(load_library().wkv_forward_infer(_DTYPE_CODE[k.dtype], B, T, C, _ptr(w), _ptr(u),
                                            _ptr(k), _ptr(v), _ptr(r), _ptr(y), _ptr(st[0]),
                                            _ptr(st[1]), _ptr(st[2]), _ptr(workspace),
                                            workspace.numel(), _stream(dev)))
    return y


def forward_gated(w, u, k, v, r, workspace=None, out=None):
    """sigma(r) * WKV(w, u, k, v) [B,T,C], the receptance-gated output (y is not written).
    Formats as for forward()."""
    return _forward_common(w, u, k, v, r, workspace, out)


def backward_gated(w, u, k, v, r, dout, fwd_workspace=None, workspace=None, out=None):
    """(dk, dv, dr, dw, du) of sum(dout * sigma(r) * y). `fwd_workspace` as for backward();
    `out` may hold preallocated (dk, dv, dr, dw, du). Formats as for backward()."""
    return _backward_common(w, u, k, v, dout, r, fwd_workspace, workspace, out)


def decode_step(w, u, k, v, a, b, p, out=None):
    """One token for B sequences: y [B,C]; the state (a, b, p) [B,C] float32 is updated in
    place. k, v (and y / out) share one of float32, bfloat16, float16."""
    if not isinstance(k, torch.Tensor):
        raise TypeError("k must be a torch.Tensor")
    if k.dtype not in _DTYPE_CODE:
        raise TypeError("k must be float32, bfloat16 or float16, got %s" % k.dtype)
    _need(k, "k", 2, dtype=k.dtype)
    dev = k.device
    _need(v, "v", 2, dev, dtype=k.dtype)
    for t, n in ((v, "v"), (a, "a"), (b, "b"), (p, "p")):
        if n != "v":
            _need(t, n, 2, dev)
        if t.shape != k.shape:
            raise ValueError("%s shape %s != k shape %s" % (n, tuple(t.shape), tuple(k.shape)))
    _need(w, "w", 1, dev)
    _need(u, "u", 1, dev)
    B, C = k.shape
    if w.shape[0] != C or u.shape[0] != C:
        raise ValueError("w and u must have C=%d elements" % C)
    y = torch.empty_like(k) if out is None else out
    _need(y, "out", 2, dev, dtype=k.dtype)
    if y.shape != k.shape:
        raise ValueError("out has the wrong shape")
    lib = load_library()
    if k.dtype == torch.float32:
        rc = lib.wkv_decode_step(B, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
                                 _ptr(p), _ptr(y), _stream(dev))
    else:
        rc = lib.wkv_decode_step_typed(_DTYPE_CODE[k.dtype], B, C, _ptr(w), _ptr(u), _ptr(k),
                                       _ptr(v), _ptr(a), _ptr(b), _ptr(p), _ptr(y),
                                       _stream(dev))
    _check(rc)
    return y


def _check_shift(x, mu, x_prev):
    _need(x, "x", 3)
    dev = x.device
    B, T, C = x.shape
    _need(mu, "mu", 2, dev)
    if tuple(mu.shape) != (3, C):
        raise ValueError("mu must have shape (3, %d)" % C)
    if x_prev is not None:
        _need(x_prev, "x_prev", 2, dev)
        if tuple(x_prev.shape) != (B, C):
            raise ValueError("x_prev must have shape (%d, %d)" % (B, C))
    return B, T, C, dev


def token_shift(x, mu, x_prev=None):
    """The token-shift mix: out_m = mu[m] * x[t] + (1 - mu[m]) * x[t-1] for m = r, k, v
    (x[-1] = x_prev, zeros if None). Returns (out_r, out_k, out_v, x_last)."""
    B, T, C, dev = _check_shift(x, mu, x_prev)
    outs = tuple(torch.empty_like(x) for _ in range(3))
    last = torch.empty(B, C, dtype=torch.float32, device=dev)
    _check(load_library().wkv_token_shift(B, T, C, _ptr(x), _ptr(x_prev), _ptr(mu),
                                          _ptr(outs[0]), _ptr(outs[1]), _ptr(outs[2]),
                                          _ptr(last) if T > 0 else None, _stream(dev)))
    if T == 0:
        last = x_prev.clone() if x_prev is not None else torch.zeros(B, C, device=dev)
    return outs + (last,)


def token_shift_backward(x, mu, dout, x_prev=None):
    """(dx, dx_prev, dmu) of sum over m of dout[m] * out_m; dx_prev is None without x_prev
    (a fresh sequence has no previous input)."""
    B, T, C, dev = _check_shift(x, mu, x_prev)
    if len(dout) != 3:
        raise ValueError("dout must hold the three cotangents (r, k, v)")
    for t, n in zip(dout, ("dout_r", "dout_k", "dout_v")):
        _need(t, n, 3, dev)
        if t.shape != x.shape:
            raise ValueError("%s has the wrong shape" % n)
    lib = load_library()
    ws = torch.empty(max(16, int(lib.wkv_token_shift_backward_workspace_size(B, T, C))),
                     dtype=torch.uint8, device=dev)
    dx = torch.empty_like(x)
    dprev = torch.empty(B, C, dtype=torch.float32, device=dev) if x_prev is not None else None
    dmu = torch.empty(3, C, dtype=torch.float32, device=dev)
    _check(lib.wkv_token_shift_backward(B, T, C, _ptr(x), _ptr(x_prev), _ptr(mu),
                                        _ptr(dout[0]), _ptr(dout[1]), _ptr(dout[2]), _ptr(dx),
                                        _ptr(dprev), _ptr(dmu), _ptr(ws), ws.numel(),
                                        _stream(dev)))
    return dx, dprev, dmu


class WKV(torch.autograd.Function):
    """Autograd wrapper: y = WKV(w, u, k, v); the forward's workspace is kept for backward."""

    @staticmethod
    def forward(ctx, w, u, k, v):
        B, T, C = k.shape
        ws = forward_workspace(B, T, C, k.device)
        y = forward(w, u, k, v, workspace=ws)
        ctx.save_for_backward(w, u, k, v, ws)
        return y

    @staticmethod
    def backward(ctx, dy):
        w, u, k, v, ws = ctx.saved_tensors
        dk, dv, dw, du = backward(w, u, k, v, dy.contiguous(), fwd_workspace=ws)
        return dw, du, dk, dv


load_library()
