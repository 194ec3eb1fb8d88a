"""Python binding of librglru.so (include/rglru.h): argument marshalling only.

Each function takes torch tensors, checks dtype / device / contiguity, passes raw device pointers
and the current HIP stream to the C entry point of the same name, and raises RglruError on a
non-zero status. Every step of the computation runs in the library's HIP kernels; there is no
fallback of any kind: if librglru.so is missing or fails to load, importing this package fails.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "librglru.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run gated_linear_recurrence_conv1d_amd/build.py "
                      "(or __graft_entry__.build())")
_lib = ctypes.CDLL(LIB_PATH)

RGLRU_OK = 0
RGLRU_ERR_INVALID_ARG = 1
RGLRU_ERR_UNSUPPORTED = 2
RGLRU_ERR_WORKSPACE = 3
RGLRU_ERR_HIP = 4
RGLRU_F32 = 0
RGLRU_BF16 = 1
RGLRU_PLAN_AUTO = 0
RGLRU_PLAN_DIRECT = 1
RGLRU_PLAN_CHUNKED = 2
RGLRU_PLAN_FUSED = 3
_PLANS = {"auto": RGLRU_PLAN_AUTO, "direct": RGLRU_PLAN_DIRECT, "chunked": RGLRU_PLAN_CHUNKED,
          "fused": RGLRU_PLAN_FUSED}

_vp = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t

_lib.rglru_status_string.argtypes = [_i]
_lib.rglru_status_string.restype = ctypes.c_char_p
_lib.rglru_forward_workspace_size.argtypes = [_i] * 5
_lib.rglru_forward_workspace_size.restype = _sz
_lib.rglru_scan_workspace_size.argtypes = [_i] * 5
_lib.rglru_scan_workspace_size.restype = _sz
_lib.rglru_forward_workspace_size_planned.argtypes = [_i] * 7
_lib.rglru_forward_workspace_size_planned.restype = _sz
_lib.rglru_lookback_failures.argtypes = [_vp, _sz, ctypes.POINTER(ctypes.c_uint), _vp]
_lib.rglru_lookback_failures.restype = _i
_lib.rglru_forward_plan_info.argtypes = [_i] * 5 + [ctypes.POINTER(_i), ctypes.POINTER(_i)]
_lib.rglru_forward_plan_info.restype = _i
_lib.rglru_forward.argtypes = [_vp] * 10 + [_i] * 5 + [_vp, _sz, _vp]
_lib.rglru_forward.restype = _i
_lib.rglru_forward_noalloc.argtypes = [_vp] * 10 + [_i] * 5 + [_vp]
_lib.rglru_forward_noalloc.restype = _i
_lib.rglru_forward_noalloc_max_bytes.argtypes = []
_lib.rglru_forward_noalloc_max_bytes.restype = _sz
_lib.rglru_forward_planned.argtypes = [_vp] * 10 + [_i] * 5 + [_vp, _sz, _vp, _i, _i]
_lib.rglru_forward_planned.restype = _i
_lib.rglru_gate_preacts.argtypes = [_vp] * 7 + [_i] * 5 + [_vp]
_lib.rglru_gate_preacts.restype = _i
_lib.rglru_scan_preacts.argtypes = [_vp] * 7 + [_i] * 5 + [_vp, _sz, _vp, _i, _i]
_lib.rglru_scan_preacts.restype = _i
_lib.rglru_decode_step.argtypes = [_vp] * 10 + [_i] * 4 + [_vp]
_lib.rglru_decode_step.restype = _i
_lib.rglru_prefill_state.argtypes = [_vp, _vp] + [_i] * 4 + [_vp]
_lib.rglru_prefill_state.restype = _i
_lib.rglru_local_mqa.argtypes = [_vp] * 4 + [_i] * 5 + [ctypes.c_float, _i, _vp]
_lib.rglru_local_mqa.restype = _i
_lib.rglru_backward_workspace_size.argtypes = [_i] * 5
_lib.rglru_backward_workspace_size.restype = _sz
_lib.rglru_backward.argtypes = [_vp] * 19 + [_i] * 5 + [_vp, _sz, _vp]
_lib.rglru_backward.restype = _i


class RglruError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {rglru_status_string(status)} (status {status})")
        self.status = status


def rglru_status_string(status: int) -> str:
    return _lib.rglru_status_string(int(status)).decode()


def _dt(dtype) -> int:
    if dtype in (torch.bfloat16, "bf16", RGLRU_BF16):
        return RGLRU_BF16
    if dtype in (torch.float32, "f32", RGLRU_F32):
        return RGLRU_F32
    raise ValueError(f"unsupported dtype {dtype}")


def _ptr(t, io_dtype=None, name=""):
    """Raw device pointer of a contiguous CUDA (HIP) tensor, or None."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if io_dtype is not None and t.dtype != io_dtype:
        raise ValueError(f"{name}: expected {io_dtype}, got {t.dtype}")
    return t.data_ptr()


def _shape(t, shape, name):
    """Raise ValueError unless tensor t (if given) has exactly this shape. Every buffer's size is
    checked here, before any call: the C ABI takes sizes only through B, T, D, H, N, so a tensor
    of another size would be read or written out of its bounds on the device."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


def _dims(x, W_a):
    if x.dim() != 3:
        raise ValueError(f"x: expected [B, T, D], got shape {tuple(x.shape)}")
    B, T, D = x.shape
    if W_a.dim() != 3 or W_a.shape[0] < 1 or D % W_a.shape[0]:
        raise ValueError(f"W_a: expected [H, D/H, D/H] with D = {D}, got {tuple(W_a.shape)}")
    return B, T, D, W_a.shape[0]


def _check_params(D, H, conv_w, W_a, b_a, W_x, b_x, Lam):
    Dh = D // H
    _shape(conv_w, (4, D), "conv_w")
    _shape(W_a, (H, Dh, Dh), "W_a")
    _shape(W_x, (H, Dh, Dh), "W_x")
    _shape(b_a, (D,), "b_a")
    _shape(b_x, (D,), "b_x")
    _shape(Lam, (D,), "Lambda")


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(status, where):
    if status != RGLRU_OK:
        raise RglruError(status, where)


def rglru_forward_workspace_size(B, T, D, H, dtype) -> int:
    return int(_lib.rglru_forward_workspace_size(B, T, D, H, _dt(dtype)))


def rglru_scan_workspace_size(B, T, D, H, dtype) -> int:
    return int(_lib.rglru_scan_workspace_size(B, T, D, H, _dt(dtype)))


def rglru_forward_workspace_size_planned(B, T, D, H, dtype, plan="auto", chunk_len=0) -> int:
    return int(_lib.rglru_forward_workspace_size_planned(B, T, D, H, _dt(dtype), _PLANS[plan],
                                                         int(chunk_len)))


def rglru_lookback_failures(workspace, stream=None) -> int:
    """Look-back waits of the last forward / backward call on `workspace` that gave up (0 after
    a normal call). Waits for the stream."""
    n = ctypes.c_uint(0)
    _check(_lib.rglru_lookback_failures(_ptr(workspace, None, "workspace"),
                                        workspace.numel() * workspace.element_size(),
                                        ctypes.byref(n), _stream(stream)),
           "rglru_lookback_failures")
    return int(n.value)


def rglru_forward_plan_info(B, T, D, H, dtype):
    plan, chunk = _i(), _i()
    _check(_lib.rglru_forward_plan_info(B, T, D, H, _dt(dtype), ctypes.byref(plan),
                                        ctypes.byref(chunk)), "rglru_forward_plan_info")
    return {RGLRU_PLAN_DIRECT: "direct", RGLRU_PLAN_CHUNKED: "chunked",
            RGLRU_PLAN_FUSED: "fused"}[plan.value], chunk.value


def _fwd_args(x, conv_w, W_a, b_a, W_x, b_x, Lam, h0, y, h_T):
    io = x.dtype
    B, T, D, H = _dims(x, W_a)
    _check_params(D, H, conv_w, W_a, b_a, W_x, b_x, Lam)
    _shape(h0, (B, D), "h0")
    _shape(y, (B, T, D), "y")
    _shape(h_T, (B, D), "h_T")
    f32 = torch.float32
    ptrs = [_ptr(x, io, "x"), _ptr(conv_w, io, "conv_w"), _ptr(W_a, io, "W_a"),
            _ptr(b_a, f32, "b_a"), _ptr(W_x, io, "W_x"), _ptr(b_x, f32, "b_x"),
            _ptr(Lam, f32, "Lambda"), _ptr(h0, f32, "h0"), _ptr(y, io, "y"),
            _ptr(h_T, f32, "h_T")]
    return ptrs, (B, T, D, H, _dt(io))


def rglru_forward(x, conv_w, W_a, b_a, W_x, b_x, Lambda, h0, y, h_T, workspace, stream=None):
    ptrs, dims = _fwd_args(x, conv_w, W_a, b_a, W_x, b_x, Lambda, h0, y, h_T)
    _check(_lib.rglru_forward(*ptrs, *dims, _ptr(workspace, None, "workspace"),
                              workspace.numel() * workspace.element_size(), _stream(stream)),
           "rglru_forward")


def rglru_forward_noalloc(x, conv_w, W_a, b_a, W_x, b_x, Lambda, h0, y, h_T, stream=None):
    """rglru_forward with the library's own fixed device workspace (no allocation)."""
    ptrs, dims = _fwd_args(x, conv_w, W_a, b_a, W_x, b_x, Lambda, h0, y, h_T)
    _check(_lib.rglru_forward_noalloc(*ptrs, *dims, _stream(stream)), "rglru_forward_noalloc")


def rglru_forward_noalloc_max_bytes() -> int:
    return int(_lib.rglru_forward_noalloc_max_bytes())


def rglru_forward_planned(x, conv_w, W_a, b_a, W_x, b_x, Lambda, h0, y, h_T, workspace,
                          plan="auto", chunk_len=0, stream=None):
    ptrs, dims = _fwd_args(x, conv_w, W_a, b_a, W_x, b_x, Lambda, h0, y, h_T)
    _check(_lib.rglru_forward_planned(*ptrs, *dims, _ptr(workspace, None, "workspace"),
                                      workspace.numel() * workspace.element_size(),
                                      _stream(stream), _PLANS[plan], int(chunk_len)),
           "rglru_forward_planned")


def rglru_gate_preacts(x, conv_w, W_a, b_a, W_x, b_x, pre, stream=None):
    """pre: int32 [B,T,D] (fp16 pairs) for bf16 x, float32 [B,T,D,2] for fp32 x."""
    io = x.dtype
    B, T, D, H = _dims(x, W_a)
    _check_params(D, H, conv_w, W_a, b_a, W_x, b_x, None)
    _check_pre(pre, x)
    f32 = torch.float32
    _check(_lib.rglru_gate_preacts(_ptr(x, io, "x"), _ptr(conv_w, io, "conv_w"),
                                   _ptr(W_a, io, "W_a"), _ptr(b_a, f32, "b_a"),
                                   _ptr(W_x, io, "W_x"), _ptr(b_x, f32, "b_x"),
                                   _ptr(pre, None, "pre"), B, T, D, H, _dt(io), _stream(stream)),
           "rglru_gate_preacts")


def _check_pre(pre, x):
    B, T, D = x.shape
    if x.dtype == torch.bfloat16:
        _shape(pre, (B, T, D), "pre")
        if pre.dtype != torch.int32:
            raise ValueError("pre: expected int32 (fp16 pairs) for bf16 x")
    else:
        _shape(pre, (B, T, D, 2), "pre")
        if pre.dtype != torch.float32:
            raise ValueError("pre: expected float32 pairs for fp32 x")


def rglru_scan_preacts(x, pre, conv_w, Lambda, h0, y, h_T, H, workspace=None, plan="auto",
                       chunk_len=0, stream=None):
    io = x.dtype
    if x.dim() != 3:
        raise ValueError(f"x: expected [B, T, D], got shape {tuple(x.shape)}")
    B, T, D = x.shape
    if H < 1 or D % H:
        raise ValueError(f"H = {H} must divide D = {D}")
    _check_pre(pre, x)
    _shape(conv_w, (4, D), "conv_w")
    _shape(Lambda, (D,), "Lambda")
    _shape(h0, (B, D), "h0")
    _shape(y, (B, T, D), "y")
    _shape(h_T, (B, D), "h_T")
    f32 = torch.float32
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.rglru_scan_preacts(_ptr(x, io, "x"), _ptr(pre, None, "pre"),
                                   _ptr(conv_w, io, "conv_w"), _ptr(Lambda, f32, "Lambda"),
                                   _ptr(h0, f32, "h0"), _ptr(y, io, "y"), _ptr(h_T, f32, "h_T"),
                                   B, T, D, H, _dt(io), _ptr(workspace, None, "workspace"), wsb,
                                   _stream(stream), _PLANS[plan], int(chunk_len)),
           "rglru_scan_preacts")


def rglru_decode_step(x_t, conv_state, h, y_t, conv_w, W_a, b_a, W_x, b_x, Lambda, stream=None):
    io = x_t.dtype
    if x_t.dim() != 2:
        raise ValueError(f"x_t: expected [N, D], got shape {tuple(x_t.shape)}")
    N, D = x_t.shape
    if W_a.dim() != 3 or W_a.shape[0] < 1 or D % W_a.shape[0]:
        raise ValueError(f"W_a: expected [H, D/H, D/H] with D = {D}, got {tuple(W_a.shape)}")
    H = W_a.shape[0]
    _check_params(D, H, conv_w, W_a, b_a, W_x, b_x, Lambda)
    _shape(conv_state, (N, 3, D), "conv_state")
    _shape(h, (N, D), "h")
    _shape(y_t, (N, D), "y_t")
    f32 = torch.float32
    _check(_lib.rglru_decode_step(_ptr(x_t, io, "x_t"), _ptr(conv_state, io, "conv_state"),
                                  _ptr(h, f32, "h"), _ptr(y_t, io, "y_t"),
                                  _ptr(conv_w, io, "conv_w"), _ptr(W_a, io, "W_a"),
                                  _ptr(b_a, f32, "b_a"), _ptr(W_x, io, "W_x"),
                                  _ptr(b_x, f32, "b_x"), _ptr(Lambda, f32, "Lambda"), N, D, H,
                                  _dt(io), _stream(stream)),
           "rglru_decode_step")


def rglru_prefill_state(x, conv_state, stream=None):
    """conv_state [B,3,D] (x's dtype) = the last three inputs of each sequence of x [B,T,D]."""
    io = x.dtype
    if x.dim() != 3:
        raise ValueError(f"x: expected [B, T, D], got shape {tuple(x.shape)}")
    B, T, D = x.shape
    _shape(conv_state, (B, 3, D), "conv_state")
    _check(_lib.rglru_prefill_state(_ptr(x, io, "x"), _ptr(conv_state, io, "conv_state"), B, T, D,
                                    _dt(io), _stream(stream)), "rglru_prefill_state")


def prefill_state(x, stream=None):
    """A new conv-state tensor [B,3,D] for continuing x [B,T,D] with decode steps."""
    B, T, D = x.shape
    cs = torch.empty((B, 3, D), dtype=x.dtype, device=x.device)
    rglru_prefill_state(x, cs, stream)
    return cs


def rglru_local_mqa(q, k, v, o, window, scale=0.0, stream=None):
    """q, o [B,T,Hq,dh]; k, v [B,T,dh]; bf16."""
    if q.dim() != 4:
        raise ValueError(f"q: expected [B, T, Hq, dh], got shape {tuple(q.shape)}")
    B, T, Hq, dh = q.shape
    _shape(k, (B, T, dh), "k")
    _shape(v, (B, T, dh), "v")
    _shape(o, (B, T, Hq, dh), "o")
    bf = torch.bfloat16
    _check(_lib.rglru_local_mqa(_ptr(q, bf, "q"), _ptr(k, bf, "k"), _ptr(v, bf, "v"),
                                _ptr(o, bf, "o"), B, T, Hq, dh, int(window), float(scale),
                                RGLRU_BF16, _stream(stream)), "rglru_local_mqa")


def local_mqa(q, k, v, window, scale=0.0, stream=None):
    """Returns o [B,T,Hq,dh] (bf16)."""
    o = torch.empty_like(q)
    rglru_local_mqa(q, k, v, o, window, scale, stream)
    return o


def rglru_backward_workspace_size(B, T, D, H, dtype) -> int:
    return int(_lib.rglru_backward_workspace_size(B, T, D, H, _dt(dtype)))


def rglru_backward(x, conv_w, W_a, b_a, W_x, b_x, Lambda, h0, y, dy, dh_T, dx, dconv_w, dW_a,
                   db_a, dW_x, db_x, dLambda, dh0, workspace, stream=None):
    io = x.dtype
    B, T, D, H = _dims(x, W_a)
    Dh = D // H
    _check_params(D, H, conv_w, W_a, b_a, W_x, b_x, Lambda)
    for t, shape, name in ((h0, (B, D), "h0"), (y, (B, T, D), "y"), (dy, (B, T, D), "dy"),
                           (dh_T, (B, D), "dh_T"), (dx, (B, T, D), "dx"),
                           (dconv_w, (4, D), "dconv_w"), (dW_a, (H, Dh, Dh), "dW_a"),
                           (db_a, (D,), "db_a"), (dW_x, (H, Dh, Dh), "dW_x"), (db_x, (D,), "db_x"),
                           (dLambda, (D,), "dLambda"), (dh0, (B, D), "dh0")):
        _shape(t, shape, name)
    f32 = torch.float32
    ptrs = [_ptr(x, io, "x"), _ptr(conv_w, io, "conv_w"), _ptr(W_a, io, "W_a"),
            _ptr(b_a, f32, "b_a"), _ptr(W_x, io, "W_x"), _ptr(b_x, f32, "b_x"),
            _ptr(Lambda, f32, "Lambda"), _ptr(h0, f32, "h0"), _ptr(y, io, "y"),
            _ptr(dy, io, "dy"), _ptr(dh_T, f32, "dh_T"), _ptr(dx, io, "dx"),
            _ptr(dconv_w, f32, "dconv_w"), _ptr(dW_a, f32, "dW_a"), _ptr(db_a, f32, "db_a"),
            _ptr(dW_x, f32, "dW_x"), _ptr(db_x, f32, "db_x"), _ptr(dLambda, f32, "dLambda"),
            _ptr(dh0, f32, "dh0")]
    _check(_lib.rglru_backward(*ptrs, B, T, D, H, _dt(io), _ptr(workspace, None, "workspace"),
                               workspace.numel() * workspace.element_size(), _stream(stream)),
           "rglru_backward")


# ---- convenience wrappers (allocate outputs with torch, then call the entry points above) ----
def pre_buffer(x):
    """An empty pre-activation buffer in the layout rglru_gate_preacts writes."""
    B, T, D = x.shape
    if x.dtype == torch.bfloat16:
        return torch.empty((B, T, D), dtype=torch.int32, device=x.device)
    return torch.empty((B, T, D, 2), dtype=torch.float32, device=x.device)


def forward(x, conv_w, W_a, b_a, W_x, b_x, Lambda, h0=None, plan="auto", chunk_len=0,
            workspace=None, stream=None):
    """Returns (y, h_T)."""
    B, T, D = x.shape
    H = W_a.shape[0]
    y = torch.empty_like(x)
    h_T = torch.empty((B, D), dtype=torch.float32, device=x.device)
    if workspace is None:
        n = rglru_forward_workspace_size_planned(B, T, D, H, x.dtype, plan, chunk_len)
        if n == 0:
            raise RglruError(RGLRU_ERR_UNSUPPORTED if plan == "fused" else RGLRU_ERR_INVALID_ARG,
                             "rglru_forward_workspace_size_planned")
        workspace = torch.empty(n, dtype=torch.uint8, device=x.device)
    rglru_forward_planned(x, conv_w, W_a, b_a, W_x, b_x, Lambda, h0, y, h_T, workspace, plan,
                          chunk_len, stream)
    return y, h_T


def decode_step(x_t, conv_state, h, conv_w, W_a, b_a, W_x, b_x, Lambda, stream=None):
    """In place on conv_state and h; returns y_t."""
    y_t = torch.empty_like(x_t)
    rglru_decode_step(x_t, conv_state, h, y_t, conv_w, W_a, b_a, W_x, b_x, Lambda, stream)
    return y_t


def backward(x, conv_w, W_a, b_a, W_x, b_x, Lambda, h0, y, dy, dh_T=None, want_dh0=True,
             workspace=None, stream=None):
    """Gradients through the forward. Returns a dict with dx (x's dtype) and fp32 dconv_w [4,D],
    dW_a, dW_x [H,Dh,Dh], db_a, db_x, dLam [D] and dh0 [B,D] (None unless want_dh0)."""
    B, T, D = x.shape
    H = W_a.shape[0]
    Dh = D // H
    dev = x.device
    f32 = torch.float32
    out = {"dx": torch.empty_like(x), "dconv_w": torch.empty((4, D), dtype=f32, device=dev),
           "dW_a": torch.empty((H, Dh, Dh), dtype=f32, device=dev),
           "db_a": torch.empty(D, dtype=f32, device=dev),
           "dW_x": torch.empty((H, Dh, Dh), dtype=f32, device=dev),
           "db_x": torch.empty(D, dtype=f32, device=dev),
           "dLam": torch.empty(D, dtype=f32, device=dev),
           "dh0": torch.empty((B, D), dtype=f32, device=dev) if want_dh0 else None}
    if workspace is None:
        workspace = torch.empty(rglru_backward_workspace_size(B, T, D, H, x.dtype),
                                dtype=torch.uint8, device=dev)
    rglru_backward(x, conv_w, W_a, b_a, W_x, b_x, Lambda, h0, y, dy, dh_T, out["dx"],
                   out["dconv_w"], out["dW_a"], out["db_a"], out["dW_x"], out["db_x"],
                   out["dLam"], out["dh0"], workspace, stream)
    return out
