"""fp64 CPU oracle for local (sliding-window) multi-query attention.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may use it; it never imports the product and the product never imports it.

What it computes (alby13 blog "Beyond Transformer Architecture: Griffin and Google RecurrentGemma",
section "Core Components of Griffin -- 2. Local Sliding-Window MQA": Griffin's attention is
multi-query -- every query head shares one key/value head -- and each position attends only within
a fixed window, typically 1024 tokens, which bounds the KV cache; Soham De's Griffin thread, tweet
on adding a local attention block every two recurrent blocks: it captures the recent past).

For every sequence b, query head h and position t, with the window [lo_t, t], lo_t = max(0, t-W+1):
    s_u = scale * <q[b,t,h,:], k[b,u,:]>          for u in [lo_t, t]
    p_u = exp(s_u - max_u s_u) / sum_u exp(s_u - max_u s_u)
    o[b,t,h,:] = sum_u p_u v[b,u,:]
scale = 1/sqrt(dh) unless given. Readings where the pages are silent (each listed in the design
notes): the window holds W positions including t itself; no positional encoding and no logit
cap; causal (no position attends to later ones).

Shapes: q [B, T, Hq, dh], k and v [B, T, dh]; returns o [B, T, Hq, dh] as float64. The whole
softmax row is formed with numpy matmuls and reductions (library primitives), one (b, h) at a
time, in blocks of query rows to bound memory.
"""
from __future__ import annotations

import numpy as np


def local_mqa(q, k, v, window, scale=None, block=512):
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, T, Hq, dh = q.shape
    assert k.shape == (B, T, dh) and v.shape == (B, T, dh) and window >= 1
    if scale is None:
        scale = 1.0 / np.sqrt(dh)
    o = np.empty((B, T, Hq, dh), np.float64)
    pos = np.arange(T)
    for b in range(B):
        for t0 in range(0, T, block):
            t1 = min(T, t0 + block)
            u0 = max(0, t0 - window + 1)  # first key any row of this block can see
            keys = k[b, u0:t1]            # [U, dh]
            vals = v[b, u0:t1]
            tt = pos[t0:t1, None]
            uu = pos[None, u0:t1]
            visible = (uu <= tt) & (uu > tt - window)  # [rows, U]
            for h in range(Hq):
                s = scale * (q[b, t0:t1, h] @ keys.T)  # [rows, U]
                s = np.where(visible, s, -np.inf)
                s -= s.max(axis=1, keepdims=True)
                p = np.exp(s)
                p /= p.sum(axis=1, keepdims=True)
                o[b, t0:t1, h] = p @ vals
    return o


def local_mqa_rows(q, k, v, window, rows, scale=None):
    """o for a list of (b, t, h) triples only, each computed on its own (for sampled checks of
    full-size outputs). Returns [len(rows), dh]."""
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    dh = q.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(dh)
    out = np.empty((len(rows), dh), np.float64)
    for i, (b, t, h) in enumerate(rows):
        lo = max(0, t - window + 1)
        keys = k[b, lo:t + 1].astype(np.float64)
        s = scale * (keys @ q[b, t, h].astype(np.float64))
        s -= s.max()
        p = np.exp(s)
        p /= p.sum()
        out[i] = p @ v[b, lo:t + 1].astype(np.float64)
    return out
