"""Pins of the oracle's backward (CPU): every gradient against central finite differences of the
oracle's forward, which tests/test_oracle_pins.py pins to the method's definition. The loss is
L = sum(dy * y) + sum(dh_T * h_T) with random weights dy, dh_T. Small shapes (a few hundred
parameters, each perturbed twice), three regimes: generic gates, the recurrence gate closed
exactly (r = 0, a = 1, m = 0: the normaliser's derivative at its limit) and fast decay."""
import numpy as np
import pytest

import oracle


def setup(seed, B=2, T=9, D=8, H=2, closed=False, fast=False):
    rng = np.random.default_rng(seed)
    Dh = D // H
    p = {
        "x": rng.standard_normal((B, T, D)),
        "conv_w": rng.standard_normal((4, D)) * 0.5,
        "W_a": rng.standard_normal((H, Dh, Dh)) / np.sqrt(Dh),
        "b_a": rng.standard_normal(D) * 0.5,
        "W_x": rng.standard_normal((H, Dh, Dh)) / np.sqrt(Dh),
        "b_x": rng.standard_normal(D) * 0.5,
        "Lam": rng.uniform(2.0, 7.0, D),
        "h0": rng.standard_normal((B, D)) * 0.3,
    }
    if closed:
        p["W_a"][:] = 0.0
        p["b_a"][:] = -1e4          # r = 0 exactly: a = 1, m = 0
    if fast:
        p["Lam"] = rng.uniform(-3.0, 0.0, D)  # a^c in (0.0003, 0.5): decays of a few steps
    dy = rng.standard_normal((B, T, D))
    dh_T = rng.standard_normal((B, D))
    return p, dy, dh_T


def loss(p, dy, dh_T):
    y, hT = oracle.forward(p["x"], p["conv_w"], p["W_a"], p["b_a"], p["W_x"], p["b_x"], p["Lam"],
                           p["h0"])
    return float(np.sum(dy * y) + np.sum(dh_T * hT))


def fd_grad(p, name, dy, dh_T, skip=None):
    base = p[name]
    g = np.zeros_like(base)
    flat = base.reshape(-1)
    gf = g.reshape(-1)
    for k in range(flat.size):
        if skip is not None and skip(k):
            continue
        v = flat[k]
        eps = 1e-6 * max(1.0, abs(v))
        flat[k] = v + eps
        lp = loss(p, dy, dh_T)
        flat[k] = v - eps
        lm = loss(p, dy, dh_T)
        flat[k] = v
        gf[k] = (lp - lm) / (2 * eps)
    return g


GRADS = {"x": "dx", "conv_w": "dconv_w", "W_a": "dW_a", "b_a": "db_a", "W_x": "dW_x",
         "b_x": "db_x", "Lam": "dLam", "h0": "dh0"}


@pytest.mark.parametrize("regime", ["generic", "closed", "fast"])
def test_gradients_match_finite_differences(regime):
    p, dy, dh_T = setup(11, closed=regime == "closed", fast=regime == "fast")
    g = oracle.backward(p["x"], p["conv_w"], p["W_a"], p["b_a"], p["W_x"], p["b_x"], p["Lam"],
                        p["h0"], dy, dh_T)
    for name, gname in GRADS.items():
        fd = fd_grad(p, name, dy, dh_T)
        scale = max(float(np.max(np.abs(fd))), 1e-12)
        e = float(np.max(np.abs(g[gname] - fd))) / scale
        assert e < 2e-6, (regime, name, e)


def test_closed_gate_gradients_are_exact():
    """With r = 0 the state never moves: y_t = h0 for all t. So dh0 = sum_t dy_t + dh_T exactly,
    and nothing reaches x, the conv, the input gate or Lambda (the a = 1 limit)."""
    p, dy, dh_T = setup(3, closed=True)
    g = oracle.backward(p["x"], p["conv_w"], p["W_a"], p["b_a"], p["W_x"], p["b_x"], p["Lam"],
                        p["h0"], dy, dh_T)
    assert np.allclose(g["dh0"], dy.sum(axis=1) + dh_T, rtol=1e-14, atol=1e-13)
    for k in ("dx", "dconv_w", "dW_x", "db_x", "dLam", "dW_a", "db_a"):
        assert np.all(g[k] == 0.0), k


def test_decay_zero_gradients_closed_form():
    """Lambda = -1e4 gives a = 0 exactly: y_t = sigmoid(px_t) * xc_t, independent of h0. With
    W_x = 0, conv_w = e_3 (xc = x) and b_x = beta: dx = dy * sigmoid(beta), dh0 = 0,
    db_x = sum_t dy * x * s (1 - s)."""
    p, dy, _ = setup(5)
    p["Lam"][:] = -1e4
    p["W_x"][:] = 0.0
    p["conv_w"][:] = 0.0
    p["conv_w"][3] = 1.0
    s = 1.0 / (1.0 + np.exp(-p["b_x"]))
    g = oracle.backward(p["x"], p["conv_w"], p["W_a"], p["b_a"], p["W_x"], p["b_x"], p["Lam"],
                        p["h0"], dy, None)
    assert np.allclose(g["dx"], dy * s, rtol=1e-13, atol=1e-14)
    assert np.all(g["dh0"] == 0.0)
    assert np.allclose(g["db_x"], np.sum(dy * p["x"] * s * (1 - s), axis=(0, 1)), rtol=1e-12)


def test_linear_in_dy_and_batch_separable():
    """Gradients are linear in (dy, dh_T) and the activations' gradients of one sequence do not
    depend on another sequence's dy."""
    p, dy, dh_T = setup(7, B=3)
    f = lambda a, b: oracle.backward(p["x"], p["conv_w"], p["W_a"], p["b_a"], p["W_x"], p["b_x"],
                                     p["Lam"], p["h0"], a, b)
    g1, g2 = f(dy, dh_T), f(2.0 * dy, 2.0 * dh_T)
    for k in GRADS.values():
        assert np.allclose(g2[k], 2.0 * g1[k], rtol=1e-12, atol=1e-14), k
    dy2 = dy.copy()
    dy2[2] = 0.0
    g3 = f(dy2, dh_T)
    assert np.array_equal(g3["dx"][:2], g1["dx"][:2])
    assert np.array_equal(g3["dh0"][:2], g1["dh0"][:2])
