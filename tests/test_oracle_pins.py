"""Pins for the fp64 oracle: each checks it against something other than itself -- a closed form,
a special case that reduces to a library routine, an invariant of the mathematics, or brute force
by an explicit product-of-sums formula on tiny inputs. A plausible slip in the oracle (a dropped
term, a flipped sign, a reversed conv tap, a transposed gate matrix, an off-by-one in the scan,
a wrong constant) fails at least one of them; the docstring of each test says which.

Sources for the properties: the recurrence gate can drop the current input and keep the history
(Soham De's Griffin thread, tweet on adding a Recurrent Gate to LRU); the gates do not read the
recurrent state and the state has a fixed size (alby13 blog, "Core Components of Griffin -- 1.
RG-LRU"); the recurrent matrix is diagonal (Soham De's thread, tweet on S4D/LRU); a temporal
Conv1D feeds the recurrence (Soham De's thread, tweet on keeping the recurrent block simple).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import expit

import oracle
from workloads import WORKLOADS, make_inputs


def rng_inputs(B, T, D, H, seed, bias=0.0, h0=True, ac=(0.9, 0.999)):
    rng = np.random.default_rng(seed)
    Dh = D // H
    v = rng.uniform(*ac, size=D) ** (1 / 8)
    Lam = np.log(v) - np.log1p(-v)
    return dict(
        x=rng.standard_normal((B, T, D)),
        conv_w=rng.standard_normal((4, D)) * 0.5,
        W_a=rng.standard_normal((H, Dh, Dh)) / np.sqrt(Dh),
        W_x=rng.standard_normal((H, Dh, Dh)) / np.sqrt(Dh),
        b_a=rng.standard_normal(D) * bias,
        b_x=rng.standard_normal(D) * bias,
        Lam=Lam,
        h0=rng.standard_normal((B, D)) if h0 else None,
    )


def call_fwd(p):
    return oracle.forward(p["x"], p["conv_w"], p["W_a"], p["b_a"], p["W_x"], p["b_x"], p["Lam"],
                          p["h0"])


def torch_causal_conv(x, conv_w):
    """Depthwise causal conv through torch's conv1d (a cross-correlation): weight[d,0,j] = w[j,d]
    meets x[t-3+j] after 3 steps of left padding. x: [B,T,D] -> [B,T,D]."""
    xt = torch.from_numpy(np.ascontiguousarray(x.transpose(0, 2, 1)))
    w = torch.from_numpy(np.ascontiguousarray(conv_w.T))[:, None, :]
    out = F.conv1d(F.pad(xt, (3, 0)), w, groups=x.shape[2])
    return out.numpy().transpose(0, 2, 1)


def blockdiag_apply(xc, W, b):
    """out[..., g*Dh+o] = b + sum_i W[g,o,i] xc[..., g*Dh+i] via a numpy matmul per head."""
    H, Dh, _ = W.shape
    parts = [xc[..., g * Dh:(g + 1) * Dh] @ W[g].T for g in range(H)]
    return np.concatenate(parts, axis=-1) + b


def relerr(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# ---------------------------------------------------------------------------------------------
def test_p1_recurrence_gate_closed_keeps_history_exactly():
    """r = 0 (W_a = 0, b_a = -1e4): a = 1 and sqrt(1 - a^2) = 0, so the state never moves and the
    input is discarded: y_t == h0 bit for bit. Catches a sign slip in the sigmoid (r would be 1),
    a missing normaliser, or an input term that bypasses the gate."""
    p = rng_inputs(2, 37, 32, 4, seed=1)
    p["W_a"][:] = 0
    p["b_a"][:] = -1e4
    y, hT = call_fwd(p)
    assert np.array_equal(y, np.broadcast_to(p["h0"][:, None, :], y.shape))
    assert np.array_equal(hT, p["h0"])


def test_p1b_decay_parameter_to_one_keeps_history():
    """Lambda = +1e4: softplus(-Lambda) = 0, so a = 1 exactly for any r and y_t == h0. Pins the
    sign of the softplus argument (softplus(+Lambda) would give a = 0)."""
    p = rng_inputs(1, 19, 16, 2, seed=2, bias=0.5)
    p["Lam"][:] = 1e4
    y, hT = call_fwd(p)
    assert np.array_equal(y, np.broadcast_to(p["h0"][:, None, :], y.shape))


def test_p2_decay_zero_gives_gated_input():
    """Lambda = -1e4 and r = 1/2 (W_a = 0, b_a = 0): log a = -4e4, a = 0, the normaliser is 1 and
    h_t = sigma(px_t) * conv(x)_t whatever h0 is. The expected value comes from torch's conv1d,
    numpy matmuls per head and scipy's expit. Catches a reversed conv tap order, a transposed
    W_x, a dropped input-gate bias, and a scan that leaks h0."""
    p = rng_inputs(2, 29, 48, 3, seed=3, bias=0.7)
    p["W_a"][:] = 0
    p["b_a"][:] = 0
    p["Lam"][:] = -1e4
    y, hT = call_fwd(p)
    xc = torch_causal_conv(p["x"], p["conv_w"])
    px = blockdiag_apply(xc, p["W_x"], p["b_x"])
    expect = expit(px) * xc
    assert relerr(y, expect) < 1e-14
    assert relerr(hT, expect[:, -1]) < 1e-14


@pytest.mark.parametrize("ac,r_bias,T", [((0.9, 0.999), 0.3, 300), ((0.99, 0.9999), -4.0, 5000),
                                         ((0.5, 0.6), 2.0, 40)])
def test_p3_constant_input_geometric_series(ac, r_bias, T):
    """W_a = W_x = 0, per-channel constant gates, conv taps (0,0,0,1) so the conv is the identity,
    x_t = xi for t >= 0. Then a = sigma(Lambda)^(8 r) (the power form, not the oracle's log form),
    and h_t = a^(t+1) h0 + sqrt(1-a^2) i xi (1 - a^(t+1)) / (1 - a), evaluated with expm1/log1p.
    Catches a wrong c, softplus(+Lambda), a missing sqrt, r/i swapped, y = h_{t-1} (off by one),
    and cancellation in 1 - a^2 beyond fp64 rounding."""
    D, H = 24, 3
    rng = np.random.default_rng(4)
    v = rng.uniform(*ac, size=D) ** (1 / 8)
    Lam = np.log(v) - np.log1p(-v)
    b_a = r_bias + 0.1 * rng.standard_normal(D)
    b_x = rng.standard_normal(D)
    xi = rng.standard_normal(D)
    h0 = rng.standard_normal((1, D))
    x = np.broadcast_to(xi, (1, T, D)).copy()
    conv_w = np.zeros((4, D))
    conv_w[3] = 1.0
    Z = np.zeros((H, D // H, D // H))
    y, hT = oracle.forward(x, conv_w, Z, b_a, Z, b_x, Lam, h0)

    r = expit(b_a)
    ig = expit(b_x)
    log_a = 8.0 * r * np.log(expit(Lam))          # log of sigma(Lambda)^(8 r)
    a = np.exp(log_a)
    m = np.sqrt(-np.expm1(2.0 * log_a))           # sqrt(1 - a^2) without cancellation
    k = np.arange(1, T + 1)[:, None]
    geo = np.expm1(k * log_a) / np.expm1(log_a)   # (1 - a^k) / (1 - a)
    expect = np.exp(k * log_a) * h0 + m * ig * xi * geo
    assert relerr(y[0], expect) < 1e-9
    assert relerr(hT[0], expect[-1]) < 1e-9


def brute_force(p):
    """h_t = (prod_{u<=t} a_u) h0 + sum_{s<=t} (prod_{s<u<=t} a_u) m_s i_s xc_s by explicit
    products and sums (no recurrence), with gates from library routines and a = sigma(Lambda)^(8r).
    """
    x = p["x"]
    B, T, D = x.shape
    xc = torch_causal_conv(x, p["conv_w"])
    r = expit(blockdiag_apply(xc, p["W_a"], p["b_a"]))
    ig = expit(blockdiag_apply(xc, p["W_x"], p["b_x"]))
    a = expit(p["Lam"]) ** (8.0 * r)
    m = np.sqrt(1.0 - a ** 2)
    h0 = p["h0"] if p["h0"] is not None else np.zeros((B, D))
    y = np.zeros((B, T, D))
    for t in range(T):
        acc = np.prod(a[:, :t + 1], axis=1) * h0
        for s in range(t + 1):
            acc = acc + np.prod(a[:, s + 1:t + 1], axis=1) * m[:, s] * ig[:, s] * xc[:, s]
        y[:, t] = acc
    return y


@pytest.mark.parametrize("seed,T,D,H,h0", [(5, 8, 16, 2, True), (6, 5, 12, 3, False),
                                           (7, 1, 8, 8, True), (8, 8, 6, 1, True)])
def test_p4_brute_force_small(seed, T, D, H, h0):
    """The whole oracle against the unrolled product-of-sums on T <= 8, random gates and biases,
    decays pushed into [0.3, 0.999] so that every term matters. Catches index slips in the scan
    (a_t vs a_{t-1}), in the conv halo, and in the head split of the gate matmuls."""
    p = rng_inputs(2, T, D, H, seed=seed, bias=0.5, h0=h0, ac=(0.3, 0.999))
    y, hT = call_fwd(p)
    ref = brute_force(p)
    assert relerr(y, ref) < 1e-13
    assert relerr(hT, ref[:, -1]) < 1e-13


# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("tap", [0, 1, 2, 3])
def test_conv_tap_order_one_hot(tap):
    """Dh = 1 and W_a = 1 make pa equal the conv output. With one-hot taps, conv_w[j] must pick
    x[t-3+j] and read zero before the sequence start."""
    B, T, D = 2, 11, 5
    rng = np.random.default_rng(9)
    x = rng.standard_normal((B, T, D))
    conv_w = np.zeros((4, D))
    conv_w[tap] = 1.0
    one = np.ones((D, 1, 1))
    zero = np.zeros(D)
    pa, px = oracle.preacts(x, conv_w, one, zero, one * 2.0, zero)
    shift = 3 - tap
    expect = np.zeros_like(x)
    expect[:, shift:] = x[:, :T - shift]
    assert np.array_equal(pa, expect)
    assert np.array_equal(px, 2.0 * expect)


def test_gate_matrix_orientation_and_heads():
    """W[g][o][i] maps input channel g*Dh+i to output channel g*Dh+o (out = W in): a single
    nonzero entry at (o=1, i=0) must move channel 0 into channel 1 of the same head only."""
    B, T, H, Dh = 1, 6, 2, 3
    D = H * Dh
    rng = np.random.default_rng(10)
    x = rng.standard_normal((B, T, D))
    conv_w = np.zeros((4, D))
    conv_w[3] = 1.0
    W = np.zeros((H, Dh, Dh))
    W[1, 1, 0] = 1.5
    b = np.arange(D) * 0.25
    pa, _ = oracle.preacts(x, conv_w, W, b, W, b)
    expect = np.broadcast_to(b, x.shape).copy()
    expect[..., Dh + 1] += 1.5 * x[..., Dh + 0]
    assert np.array_equal(pa, expect)


def test_preacts_match_library_matmul():
    p = rng_inputs(2, 33, 40, 5, seed=11, bias=0.3)
    pa, px = oracle.preacts(p["x"], p["conv_w"], p["W_a"], p["b_a"], p["W_x"], p["b_x"])
    xc = torch_causal_conv(p["x"], p["conv_w"])
    assert relerr(pa, blockdiag_apply(xc, p["W_a"], p["b_a"])) < 1e-13
    assert relerr(px, blockdiag_apply(xc, p["W_x"], p["b_x"])) < 1e-13


# ---------------------------------------------------------------------------------------------
def test_head_isolation_batch_independence_causality():
    """Block-diagonal gates and a depthwise conv: changing head 1 leaves head 0 bit-identical;
    batches are independent; nothing at t < t0 depends on x at t0."""
    p = rng_inputs(3, 40, 24, 3, seed=12, bias=0.2)
    y, _ = call_fwd(p)
    q = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in p.items()}
    q["x"][:, :, 8:16] += 1.0
    yq, _ = call_fwd(q)
    assert np.array_equal(y[..., :8], yq[..., :8]) and np.array_equal(y[..., 16:], yq[..., 16:])
    assert not np.array_equal(y[..., 8:16], yq[..., 8:16])
    q = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in p.items()}
    q["x"][1] *= -3.0
    yq, _ = call_fwd(q)
    assert np.array_equal(y[0], yq[0]) and np.array_equal(y[2], yq[2])
    q = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in p.items()}
    q["x"][:, 17] += 5.0
    yq, _ = call_fwd(q)
    assert np.array_equal(y[:, :17], yq[:, :17]) and not np.array_equal(y[:, 17], yq[:, 17])


def test_linear_in_h0():
    """With x fixed the gates are fixed, so h_t is affine in h0: y(2 h0) - y(0) = 2 (y(h0) - y(0)).
    Catches a state that leaks into the gates."""
    p = rng_inputs(2, 50, 16, 2, seed=13, bias=0.3)
    y1, _ = call_fwd(p)
    p2 = dict(p, h0=2.0 * p["h0"])
    y2, _ = call_fwd(p2)
    y0, _ = call_fwd(dict(p, h0=None))
    assert relerr(y2 - y0, 2.0 * (y1 - y0)) < 1e-12


# ---------------------------------------------------------------------------------------------
def test_decode_repeated_equals_forward_and_resume():
    """Fixed-size state: T decode steps from a zero conv state reproduce the forward, and a forward
    on x[:t1] followed by decode steps on x[t1:] (conv state seeded with x[t1-3:t1]) resumes it."""
    p = rng_inputs(3, 21, 16, 4, seed=14, bias=0.4)
    y, hT = call_fwd(p)
    B, T, D = p["x"].shape
    cs = np.zeros((B, 3, D))
    h = p["h0"].copy()
    for t in range(T):
        yt, cs, h = oracle.decode_step(p["x"][:, t], cs, h, p["conv_w"], p["W_a"], p["b_a"],
                                       p["W_x"], p["b_x"], p["Lam"])
        assert relerr(yt, y[:, t]) < 1e-14
    assert relerr(h, hT) < 1e-14
    t1 = 9
    y1, h1 = oracle.forward(p["x"][:, :t1], p["conv_w"], p["W_a"], p["b_a"], p["W_x"], p["b_x"],
                            p["Lam"], p["h0"])
    cs = p["x"][:, t1 - 3:t1].copy()
    h = h1
    for t in range(t1, T):
        yt, cs, h = oracle.decode_step(p["x"][:, t], cs, h, p["conv_w"], p["W_a"], p["b_a"],
                                       p["W_x"], p["b_x"], p["Lam"])
        assert relerr(yt, y[:, t]) < 1e-14


def test_decode_conv_state_shift_and_oldest_tap():
    """The conv state is oldest first and shifts to (cs1, cs2, x_t). With taps (1,0,0,0), a = 0
    (Lambda = -1e4, r = 1/2) and i = 1 (b_x = +1e4), the output is exactly the oldest cached
    input."""
    N, D, H = 4, 6, 2
    rng = np.random.default_rng(15)
    xt = rng.standard_normal((N, D))
    cs0 = rng.standard_normal((N, 3, D))
    conv_w = np.zeros((4, D))
    conv_w[0] = 1.0
    Z = np.zeros((H, D // H, D // H))
    y, cs, h = oracle.decode_step(xt, cs0, rng.standard_normal((N, D)), conv_w, Z, np.zeros(D), Z,
                                  np.full(D, 1e4), np.full(D, -1e4))
    assert np.array_equal(y, cs0[:, 0])
    assert np.array_equal(h, cs0[:, 0])
    assert np.array_equal(cs[:, 0], cs0[:, 1]) and np.array_equal(cs[:, 1], cs0[:, 2])
    assert np.array_equal(cs[:, 2], xt)


def test_workload_inputs_are_representable_and_seeded():
    """The shared generator: bf16 workloads hold bf16-representable values, draws are seeded, and
    the decay parameter lands in the configured range of sigma(Lambda)^8."""
    w = WORKLOADS["rg2b"]
    a = make_inputs(w, T=16, B=2)
    b = make_inputs(w, T=16, B=2)
    for k in ("x", "conv_w", "W_a", "W_x"):
        bits = a[k].view(np.uint32)
        assert np.all((bits & 0xFFFF) == 0), k
        assert np.array_equal(a[k], b[k])
    ac = expit(a["Lam"].astype(np.float64)) ** 8
    assert ac.min() > 0.9 - 1e-5 and ac.max() < 0.999 + 1e-5
