"""Pins of the local-MQA oracle against what the definition and the mathematics fix, independent
of the oracle's own code path:

* window >= T is plain causal attention: torch's scaled_dot_product_attention (fp64, CPU) with
  is_causal, each query head against the shared key/value head;
* window = 1: the softmax has one term, so o = v at the same position, exactly;
* identical keys: every visible key scores the same, so o[t] is the plain mean of v over the
  window [max(0, t-W+1), t] (a closed form);
* brute force with scalar Python loops (explicit exp and sums) on tiny inputs;
* rows computed one by one (local_mqa_rows) agree with the blocked form;
* the first W positions see the same keys with or without the window;
* query heads are independent (permuting heads permutes outputs).
"""
import numpy as np
import pytest
import torch

import oracle.local_mqa as om


def inputs(B, T, Hq, dh, seed=0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, Hq, dh))
    k = rng.standard_normal((B, T, dh))
    v = rng.standard_normal((B, T, dh))
    return q, k, v


@pytest.mark.parametrize("B,T,Hq,dh,W", [(2, 37, 3, 16, 37), (1, 80, 2, 8, 200)])
def test_full_window_is_causal_sdpa(B, T, Hq, dh, W):
    q, k, v = inputs(B, T, Hq, dh)
    o = om.local_mqa(q, k, v, W, block=16)
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)                      # [B, Hq, T, dh]
    kt = torch.from_numpy(k)[:, None].expand(B, Hq, T, dh).contiguous()
    vt = torch.from_numpy(v)[:, None].expand(B, Hq, T, dh).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    ref = ref.permute(0, 2, 1, 3).numpy()
    assert np.max(np.abs(o - ref)) < 1e-12


def test_window_one_returns_v():
    q, k, v = inputs(2, 20, 3, 8, seed=1)
    o = om.local_mqa(q, k, v, 1, block=7)
    assert np.array_equal(o, np.broadcast_to(v[:, :, None, :], o.shape))


@pytest.mark.parametrize("W", [1, 4, 9, 100])
def test_identical_keys_average_the_window(W):
    B, T, Hq, dh = 2, 30, 2, 6
    q, _, v = inputs(B, T, Hq, dh, seed=2)
    k = np.broadcast_to(np.linspace(-1, 1, dh), (B, T, dh)).copy()
    o = om.local_mqa(q, k, v, W, block=8)
    for t in range(T):
        lo = max(0, t - W + 1)
        mean = v[:, lo:t + 1].mean(axis=1)
        assert np.max(np.abs(o[:, t] - mean[:, None, :])) < 1e-13


def brute(q, k, v, W):
    B, T, Hq, dh = q.shape
    o = np.zeros_like(q)
    sc = 1.0 / np.sqrt(dh)
    for b in range(B):
        for t in range(T):
            for h in range(Hq):
                lo = max(0, t - W + 1)
                scores = []
                for u in range(lo, t + 1):
                    acc = 0.0
                    for i in range(dh):
                        acc += q[b, t, h, i] * k[b, u, i]
                    scores.append(acc * sc)
                mx = max(scores)
                e = [np.exp(s - mx) for s in scores]
                z = sum(e)
                for i in range(dh):
                    o[b, t, h, i] = sum(e[j] * v[b, lo + j, i] for j in range(len(e))) / z
    return o


@pytest.mark.parametrize("W", [1, 3, 6, 50])
def test_brute_force_tiny(W):
    q, k, v = inputs(2, 11, 2, 5, seed=3)
    assert np.max(np.abs(om.local_mqa(q, k, v, W, block=4) - brute(q, k, v, W))) < 1e-13


def test_rows_match_blocked_form():
    q, k, v = inputs(2, 150, 3, 16, seed=4)
    W = 40
    o = om.local_mqa(q, k, v, W, block=32)
    rows = [(0, 0, 0), (1, 39, 2), (1, 40, 1), (0, 149, 2), (1, 77, 0)]
    r = om.local_mqa_rows(q, k, v, W, rows)
    for i, (b, t, h) in enumerate(rows):
        assert np.max(np.abs(r[i] - o[b, t, h])) < 1e-13


def test_window_only_matters_beyond_w_and_heads_are_independent():
    q, k, v = inputs(1, 60, 4, 8, seed=5)
    W = 17
    o = om.local_mqa(q, k, v, W, block=16)
    full = om.local_mqa(q, k, v, 60, block=16)
    assert np.max(np.abs(o[:, :W] - full[:, :W])) < 1e-13
    assert np.max(np.abs(o[:, W:] - full[:, W:])) > 1e-3
    perm = [2, 0, 3, 1]
    op = om.local_mqa(q[:, :, perm], k, v, W, block=16)
    assert np.array_equal(op, o[:, :, perm])


# ---- planted mistakes: each must fail at least one pin -------------------------------------------
MUTANTS = {
    "window one short": ("(uu > tt - window)", "(uu > tt - window + 1)"),
    "window one long": ("(uu > tt - window)", "(uu >= tt - window)"),
    "not causal": ("(uu <= tt)", "(uu <= tt + 1)"),
    "no scale": ("s = scale * (q[b, t0:t1, h] @ keys.T)", "s = (q[b, t0:t1, h] @ keys.T)"),
    "softmax over the wrong axis": ("p /= p.sum(axis=1, keepdims=True)",
                                    "p /= p.sum(axis=0, keepdims=True)"),
    "first key too late": ("u0 = max(0, t0 - window + 1)", "u0 = max(0, t0 - window + 2)"),
}


def _load_mutant(old, new):
    import os
    import types
    src = open(os.path.join(os.path.dirname(om.__file__), "local_mqa.py")).read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("mqa_mutant")
    exec(compile(src.replace(old, new), "mqa_mutant", "exec"), mod.__dict__)
    return mod


def _pins_pass(mod):
    import warnings
    warnings.simplefilter("ignore", RuntimeWarning)  # a mutant may produce inf / nan
    try:
        q, k, v = inputs(2, 37, 3, 16)
        o = mod.local_mqa(q, k, v, 37, block=16)
        qt = torch.from_numpy(q).permute(0, 2, 1, 3)
        kt = torch.from_numpy(k)[:, None].expand(2, 3, 37, 16).contiguous()
        vt = torch.from_numpy(v)[:, None].expand(2, 3, 37, 16).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
        if not np.max(np.abs(o - ref.permute(0, 2, 1, 3).numpy())) < 1e-12:
            return False
        for W in (1, 3, 6):
            q, k, v = inputs(2, 11, 2, 5, seed=3)
            if not np.max(np.abs(mod.local_mqa(q, k, v, W, block=4) - brute(q, k, v, W))) < 1e-13:
                return False
        return True
    except Exception:
        return False


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    assert _pins_pass(om), "pins fail on the oracle itself"
    assert not _pins_pass(_load_mutant(*MUTANTS[name])), f"pins missed: {name}"
