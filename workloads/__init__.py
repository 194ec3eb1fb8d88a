"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module holds shapes, distributions and the random draws only: none of the method's
arithmetic. Both sides receive the very same host arrays (float32 arrays whose values are exactly
representable in the I/O dtype), so any difference between them is the method's, not the data's.

The pages measure on MassiveText training at sequence length 2048 and on evaluations that need
trained weights (alby13 blog, "Technical Foundations of RecurrentGemma"); neither is available,
so these seeded workloads stand in for them, with RecurrentGemma-like layer widths.

Draw order with ``numpy.random.default_rng(seed)`` (PCG64):
u (decay parameter) -> conv_w -> W_a -> W_x -> h0 -> conv_state -> x; each draw is made in
float32 (or float64 for u) and then rounded to the I/O dtype with round-to-nearest-even.

Distributions: N(0, v) names a variance v. Gate weights ~N(0, 1/Dh), conv weights ~N(0, 1/4)
(the 1/fan-in variances), biases 0, x ~N(0, 1). The decay parameter Lambda is drawn so that
sigma(Lambda)^8 ~ U[lo, hi]: u ~ U[lo, hi], v = u^(1/8), Lambda = log(v / (1 - v)).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

CONV_WIDTH = 4


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int            # batch (decode: rows N)
    T: int            # time steps (decode: number of consecutive steps)
    D: int            # channels
    H: int            # heads of the block-diagonal gates
    dtype: str        # "f32" or "bf16": dtype of x, y, conv_w, W_a, W_x, conv_state
    ac_lo: float      # sigma(Lambda)^8 ~ U[ac_lo, ac_hi]
    ac_hi: float
    h0_var: float     # 0 => h0 = 0
    decode: bool = False
    cs_var: float = 0.0

    @property
    def Dh(self) -> int:
        return self.D // self.H

    @property
    def elements(self) -> int:
        return self.B * self.T * self.D


WORKLOADS = {
    "tiny": Workload("tiny_b1_t256_d256_h16_f32", 1, 256, 256, 16, "f32", 0.9, 0.999, 0.0),
    "rg2b": Workload("rg2b_layer_b8_t2048_d2560_h10_bf16", 8, 2048, 2560, 10, "bf16", 0.9,
                     0.999, 0.0),
    "rg9b": Workload("rg9b_layer_b16_t4096_d4096_h16_bf16", 16, 4096, 4096, 16, "bf16", 0.9,
                     0.999, 0.1),
    "long": Workload("long_b1_t65536_d2560_h10_bf16", 1, 65536, 2560, 10, "bf16", 0.99, 0.9999,
                     0.0),
    "decode": Workload("decode_n1024_d4096_h16_bf16_256steps", 1024, 256, 4096, 16, "bf16", 0.9,
                       0.999, 0.1, decode=True, cs_var=0.1),
}


def round_to_dtype(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the I/O dtype (round-to-nearest-even) and return them as float32.
    Inputs are finite here."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "f32":
        return a
    if dtype != "bf16":
        raise ValueError(dtype)
    u = a.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) & np.uint32(0xFFFF0000)).view(np.float32)


def lambda_for_decay(u: np.ndarray) -> np.ndarray:
    """Lambda such that sigma(Lambda)^8 = u (input recipe only)."""
    v = np.power(np.asarray(u, np.float64), 1.0 / 8.0)
    return (np.log(v) - np.log1p(-v)).astype(np.float32)


def make_inputs(w: Workload, seed: int = 0, *, B: Optional[int] = None, T: Optional[int] = None,
                D: Optional[int] = None, H: Optional[int] = None,
                bias_var: float = 0.0) -> dict:
    """Draw one workload's inputs (optionally at overridden sizes, for the small parity cases).

    Returns float32 numpy arrays: x [B,T,D] (decode: [T,B,D], one slab per step), conv_w [4,D],
    W_a, W_x [H,Dh,Dh], b_a, b_x, Lam [D], h0 [B,D] or None, conv_state [B,3,D] (decode only).
    """
    B = w.B if B is None else B
    T = w.T if T is None else T
    D = w.D if D is None else D
    H = w.H if H is None else H
    if D % H:
        raise ValueError("D must be a multiple of H")
    Dh = D // H
    rng = np.random.default_rng(seed)
    u = rng.uniform(w.ac_lo, w.ac_hi, size=D)
    lam = lambda_for_decay(u)
    conv_w = round_to_dtype(rng.standard_normal((CONV_WIDTH, D), dtype=np.float32) * 0.5, w.dtype)
    sw = np.float32(1.0 / np.sqrt(Dh))
    W_a = round_to_dtype(rng.standard_normal((H, Dh, Dh), dtype=np.float32) * sw, w.dtype)
    W_x = round_to_dtype(rng.standard_normal((H, Dh, Dh), dtype=np.float32) * sw, w.dtype)
    h0 = None
    if w.h0_var > 0:
        h0 = (rng.standard_normal((B, D), dtype=np.float32) * np.float32(np.sqrt(w.h0_var)))
    cs = None
    if w.decode:
        cs = round_to_dtype(rng.standard_normal((B, CONV_WIDTH - 1, D), dtype=np.float32)
                            * np.float32(np.sqrt(w.cs_var)), w.dtype)
    if w.decode:
        x = round_to_dtype(rng.standard_normal((T, B, D), dtype=np.float32), w.dtype)
    else:
        x = round_to_dtype(rng.standard_normal((B, T, D), dtype=np.float32), w.dtype)
    if bias_var > 0:
        sb = np.float32(np.sqrt(bias_var))
        b_a = rng.standard_normal(D, dtype=np.float32) * sb
        b_x = rng.standard_normal(D, dtype=np.float32) * sb
    else:
        b_a = np.zeros(D, np.float32)
        b_x = np.zeros(D, np.float32)
    return dict(x=x, conv_w=conv_w, W_a=W_a, W_x=W_x, b_a=b_a, b_x=b_x, Lam=lam, h0=h0,
                conv_state=cs, B=B, T=T, D=D, H=H, dtype=w.dtype)


def make_cotangents(inp: dict, seed: int = 1) -> dict:
    """Seeded output gradients for a backward check: dy ~N(0, 1) [B,T,D] rounded to the I/O
    dtype and dh_T ~N(0, 1) [B,D] float32, drawn in that order from their own generator."""
    rng = np.random.default_rng(seed)
    B, T, D = inp["B"], inp["T"], inp["D"]
    dy = round_to_dtype(rng.standard_normal((B, T, D), dtype=np.float32), inp["dtype"])
    dh_T = rng.standard_normal((B, D), dtype=np.float32)
    return dict(dy=dy, dh_T=dh_T)


def make_attention_inputs(B: int, T: int, Hq: int, dh: int, seed: int = 0) -> dict:
    """Seeded inputs of local multi-query attention: q [B,T,Hq,dh], k and v [B,T,dh], each ~N(0,1)
    drawn in float32 in that order and rounded to bf16 (returned as float32 arrays)."""
    rng = np.random.default_rng(seed)
    q = round_to_dtype(rng.standard_normal((B, T, Hq, dh), dtype=np.float32), "bf16")
    k = round_to_dtype(rng.standard_normal((B, T, dh), dtype=np.float32), "bf16")
    v = round_to_dtype(rng.standard_normal((B, T, dh), dtype=np.float32), "bf16")
    return dict(q=q, k=k, v=v)


def to_device(inp: dict, device="cuda"):
    """torch tensors on `device` for the GPU side: I/O-dtype tensors for x, conv_w, W_a, W_x and
    conv_state (exact, since the values are already representable), float32 for the rest."""
    import torch

    io = torch.bfloat16 if inp["dtype"] == "bf16" else torch.float32
    out = {}
    for k in ("x", "conv_w", "W_a", "W_x", "conv_state"):
        if inp.get(k) is not None:
            out[k] = torch.from_numpy(inp[k]).to(device=device, dtype=io).contiguous()
    for k in ("b_a", "b_x", "Lam", "h0"):
        if inp.get(k) is not None:
            out[k] = torch.from_numpy(inp[k]).to(device=device, dtype=torch.float32).contiguous()
        else:
            out[k] = None
    return out
