"""fp64 CPU oracle for the Conv1D(width 4) -> RG-LRU hot path.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import this package. The product (``gated_linear_recurrence_conv1d_amd``)
never imports it, and it never imports the product. The arithmetic lives in ``rglru_oracle.c``
(plain C, fp64, compiled here with gcc); this module only marshals numpy arrays.

Every input is upcast exactly to float64 before the call, so the oracle sees the same values the
GPU receives (bf16 and fp32 both embed exactly in fp64).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rglru_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_rglru.so")
# A test that plants mistakes in the oracle (tests/test_oracle_mutants.py) points this at a
# mutant build; nothing else sets it.
_LIB_OVERRIDE = os.environ.get("RGLRU_ORACLE_LIB")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, OpenMP for the independent (b, head)
    loops only)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared", "-std=c11",
               "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        path = _LIB_OVERRIDE or _LIB
        if not _LIB_OVERRIDE and not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        i = ctypes.c_int
        lib.rglru_oracle_forward.argtypes = [i, i, i, i] + [dp] * 10
        lib.rglru_oracle_forward.restype = None
        lib.rglru_oracle_preacts.argtypes = [i, i, i, i] + [dp] * 8
        lib.rglru_oracle_preacts.restype = None
        lib.rglru_oracle_decode_step.argtypes = [i, i, i] + [dp] * 10
        lib.rglru_oracle_decode_step.restype = None
        lib.rglru_oracle_backward.argtypes = [i, i, i, i] + [dp] * 18
        lib.rglru_oracle_backward.restype = None
        lib.rglru_oracle_threads.argtypes = []
        lib.rglru_oracle_threads.restype = ctypes.c_int
        lib.rglru_oracle_set_threads.argtypes = [i]
        lib.rglru_oracle_set_threads.restype = None
        _lib = lib
    return _lib


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def threads() -> int:
    """Number of OpenMP threads the oracle runs with."""
    return int(_load().rglru_oracle_threads())


def set_threads(n: int) -> None:
    """Number of OpenMP threads later oracle calls use (timing control only)."""
    _load().rglru_oracle_set_threads(int(n))


def forward(x, conv_w, W_a, b_a, W_x, b_x, Lam, h0=None):
    """y[B,T,D], h_T[B,D] in float64. x: [B,T,D]; conv_w: [4,D]; W_a, W_x: [H,Dh,Dh] (out, in);
    b_a, b_x, Lam: [D]; h0: [B,D] or None (zeros)."""
    x = _f64(x)
    B, T, D = x.shape
    W_a = _f64(W_a)
    H = W_a.shape[0]
    assert W_a.shape == (H, D // H, D // H) and D % H == 0
    args = [_f64(conv_w), W_a, _f64(b_a), _f64(W_x), _f64(b_x), _f64(Lam)]
    h0a = None if h0 is None else _f64(h0)
    y = np.empty((B, T, D), np.float64)
    hT = np.empty((B, D), np.float64)
    _load().rglru_oracle_forward(B, T, D, H, _ptr(x), *[_ptr(a) for a in args], _ptr(h0a),
                                 _ptr(y), _ptr(hT))
    return y, hT


def preacts(x, conv_w, W_a, b_a, W_x, b_x):
    """Gate pre-activations (pa, px), each [B,T,D] float64."""
    x = _f64(x)
    B, T, D = x.shape
    W_a = _f64(W_a)
    H = W_a.shape[0]
    pa = np.empty((B, T, D), np.float64)
    px = np.empty((B, T, D), np.float64)
    _load().rglru_oracle_preacts(B, T, D, H, _ptr(x), _ptr(_f64(conv_w)), _ptr(W_a),
                                 _ptr(_f64(b_a)), _ptr(_f64(W_x)), _ptr(_f64(b_x)), _ptr(pa),
                                 _ptr(px))
    return pa, px


def decode_step(x_t, conv_state, h, conv_w, W_a, b_a, W_x, b_x, Lam):
    """One decode step. Returns (y_t, new_conv_state, new_h) as float64 copies; the inputs are
    not modified. x_t: [N,D]; conv_state: [N,3,D] oldest first; h: [N,D]."""
    x_t = _f64(x_t)
    N, D = x_t.shape
    W_a = _f64(W_a)
    H = W_a.shape[0]
    cs = _f64(conv_state).copy()
    hh = _f64(h).copy()
    y = np.empty((N, D), np.float64)
    _load().rglru_oracle_decode_step(N, D, H, _ptr(x_t), _ptr(cs), _ptr(hh), _ptr(y),
                                     _ptr(_f64(conv_w)), _ptr(W_a), _ptr(_f64(b_a)),
                                     _ptr(_f64(W_x)), _ptr(_f64(b_x)), _ptr(_f64(Lam)))
    return y, cs, hh


def backward(x, conv_w, W_a, b_a, W_x, b_x, Lam, h0, dy, dh_T=None):
    """Gradients of L = sum(dy * y) + sum(dh_T * h_T) through the forward, in float64:
    dict with dx [B,T,D], dconv_w [4,D], dW_a, dW_x [H,Dh,Dh], db_a, db_x, dLam [D] and dh0 [B,D]
    (None when h0 is None)."""
    x = _f64(x)
    B, T, D = x.shape
    W_a = _f64(W_a)
    H = W_a.shape[0]
    Dh = D // H
    out = {"dx": np.empty((B, T, D)), "dconv_w": np.empty((4, D)), "dW_a": np.empty((H, Dh, Dh)),
           "db_a": np.empty(D), "dW_x": np.empty((H, Dh, Dh)), "db_x": np.empty(D),
           "dLam": np.empty(D), "dh0": None if h0 is None else np.empty((B, D))}
    h0a = None if h0 is None else _f64(h0)
    dha = None if dh_T is None else _f64(dh_T)
    _load().rglru_oracle_backward(
        B, T, D, H, _ptr(x), _ptr(_f64(conv_w)), _ptr(W_a), _ptr(_f64(b_a)), _ptr(_f64(W_x)),
        _ptr(_f64(b_x)), _ptr(_f64(Lam)), _ptr(h0a), _ptr(_f64(dy)), _ptr(dha),
        _ptr(out["dx"]), _ptr(out["dconv_w"]), _ptr(out["dW_a"]), _ptr(out["db_a"]),
        _ptr(out["dW_x"]), _ptr(out["db_x"]), _ptr(out["dLam"]), _ptr(out["dh0"]))
    return out
