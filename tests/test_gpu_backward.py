"""GPU parity of the backward: rglru_backward through the C ABI against the fp64 oracle's
gradients, element by element, on the same seeded inputs and output gradients.

Bound, per gradient tensor (dx, dconv_w, dW_a, dW_x, db_a, db_x, dLambda, dh0): the error of the
forward's tests, err = max_i |g_i - ref_i| / max(|ref_i|, rms(ref)), below 1e-4 for fp32 I/O and
2e-2 for bf16 I/O. The bf16 path reads h[t-1] from the bf16 y, stores the pre-activations and
(dpa, dpx) as fp16 pairs, and runs the dx and dW contractions on fp16 operands; the recomputed gate
pre-activations, whose errors the gradients amplify, take the conv output as bf16 hi + lo. Single
elements then err by a few 1e-3 of the rms (with bf16 operands in the dW contraction, dW missed by
up to 2.5e-2 on these cases); a mistake in a gradient formula moves the error to O(1).
Exact cases: run-to-run bitwise reproducibility (fixed-order sums, no atomics), and the
workspace's prior contents having no effect.
"""
import numpy as np
import pytest
import torch

import gated_linear_recurrence_conv1d_amd as rg
import oracle
from workloads import WORKLOADS, make_cotangents, make_inputs, to_device

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
NAMES = ["dx", "dconv_w", "dW_a", "dW_x", "db_a", "db_x", "dLam", "dh0"]


def err(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    floor = max(float(np.sqrt(np.mean(ref ** 2))), 1e-30)
    return float(np.max(np.abs(y - ref) / np.maximum(np.abs(ref), floor)))


def case(dtype, B, T, D, H, seed=0, bias=0.25, h0=True):
    w = WORKLOADS["tiny"] if dtype == "f32" else WORKLOADS["rg2b"]
    inp = make_inputs(w, seed=seed, B=B, T=T, D=D, H=H, bias_var=bias)
    if h0:
        rng = np.random.default_rng(seed + 77)
        inp["h0"] = (rng.standard_normal((B, D)) * np.sqrt(0.1)).astype(np.float32)
    return inp


def run_gpu(inp, ct, dh_T=True, workspace=None, y=None):
    g = to_device(inp)
    io = g["x"].dtype
    if y is None:
        y, _ = rg.forward(g["x"], g["conv_w"], g["W_a"], g["b_a"], g["W_x"], g["b_x"], g["Lam"],
                          g["h0"])
    dy = torch.from_numpy(ct["dy"]).to("cuda", io)
    dhT = torch.from_numpy(ct["dh_T"]).cuda() if dh_T else None
    out = rg.backward(g["x"], g["conv_w"], g["W_a"], g["b_a"], g["W_x"], g["b_x"], g["Lam"],
                      g["h0"], y, dy, dhT, workspace=workspace)
    torch.cuda.synchronize()
    return {k: (None if v is None else v.float().cpu().numpy()) for k, v in out.items()}


def run_oracle(inp, ct, dh_T=True):
    return oracle.backward(inp["x"], inp["conv_w"], inp["W_a"], inp["b_a"], inp["W_x"],
                           inp["b_x"], inp["Lam"], inp["h0"], ct["dy"],
                           ct["dh_T"] if dh_T else None)


def check(got, ref, tol, names=NAMES):
    errs = {}
    for n in names:
        r = ref[n]
        if r is None:
            # no h0: the oracle returns no dh0; the GPU still returns g_0, compare it to zero-h0
            continue
        errs[n] = err(got[n], r)
    bad = {n: e for n, e in errs.items() if not e < tol}
    print("errors:", {n: f"{e:.2e}" for n, e in errs.items()}, flush=True)
    assert not bad, f"errors above {tol}: {bad} (all: {errs})"
    return errs


# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,B,T,D,H", [
    ("bf16", 2, 150, 512, 2),    # Dh 256: MFMA dxc and dW; 3 chunks, ragged tail
    ("bf16", 3, 129, 256, 2),    # Dh 128: MFMA dxc and dW
    ("bf16", 2, 200, 256, 4),    # Dh 64: MFMA dxc, vector-ALU dW
    ("bf16", 1, 70, 64, 2),      # Dh 32
    ("bf16", 2, 77, 96, 2),      # Dh 48: vector ALU throughout, bf16 I/O
    ("bf16", 2, 3, 256, 1),      # T shorter than the conv
    ("bf16", 1, 1, 512, 2),      # a single step
    ("bf16", 1, 64, 256, 1),     # exactly one chunk
    ("f32", 2, 130, 96, 3),      # fp32, Dh 32
    ("f32", 1, 65, 256, 1),      # fp32, Dh 256
    ("bf16", 2, 70, 33, 3),      # odd D: one channel per lane in the lane kernels, Dh 11
    ("f32", 1, 40, 15, 5),       # odd D, fp32, Dh 3
])
def test_backward_small_shapes(dtype, B, T, D, H):
    inp = case(dtype, B, T, D, H, seed=B * 100 + T)
    ct = make_cotangents(inp, seed=T)
    check(run_gpu(inp, ct), run_oracle(inp, ct), TOL[dtype])


def test_backward_tiny_fp32_config():
    """B=1, T=256, D=256, 16 heads of 16, fp32, h0 = 0 (the CPU-checkable forward config)."""
    inp = make_inputs(WORKLOADS["tiny"], seed=0)
    ct = make_cotangents(inp, seed=0)
    got = run_gpu(inp, ct)
    ref = run_oracle(inp, ct)
    check(got, ref, TOL["f32"])
    # no h0: dh0 is still g_0, which the oracle gives when asked with h0 = 0
    inp0 = dict(inp, h0=np.zeros((1, 256), np.float32))
    assert err(got["dh0"], run_oracle(inp0, ct)["dh0"]) < TOL["f32"]


def test_backward_without_dh_T():
    inp = case("bf16", 2, 150, 512, 2, seed=5)
    ct = make_cotangents(inp, seed=6)
    check(run_gpu(inp, ct, dh_T=False), run_oracle(inp, ct, dh_T=False), TOL["bf16"])


def test_backward_closed_gate():
    """r = 0 everywhere (W_a = 0, b_a = -1e4): a = 1, m = 0. Then h_t = h0, delta_t = dh_T +
    sum_{s >= t} dy_s, every input gradient through the normaliser vanishes: dx = 0, dW_x = 0,
    db_x = 0, dconv_w = 0, dpa = 0 (r (1 - r) = 0), so dW_a = 0, db_a = 0, dLambda = 0, and
    dh0 = dh_T + sum_t dy_t. The GPU must give those zeros exactly and dh0 to rounding."""
    inp = case("bf16", 2, 150, 512, 2, seed=9)
    inp["W_a"] = np.zeros_like(inp["W_a"])
    inp["b_a"] = np.full_like(inp["b_a"], -1e4)
    ct = make_cotangents(inp, seed=10)
    got = run_gpu(inp, ct)
    for n in ["dx", "dconv_w", "dW_a", "dW_x", "db_a", "db_x", "dLam"]:
        assert np.all(got[n] == 0.0), n
    expect = ct["dh_T"].astype(np.float64) + ct["dy"].astype(np.float64).sum(axis=1)
    assert err(got["dh0"], expect) < 1e-5


def test_backward_reproducible_and_ignores_workspace_contents():
    inp = case("bf16", 2, 150, 512, 2, seed=11)
    ct = make_cotangents(inp, seed=12)
    n = rg.rglru_backward_workspace_size(2, 150, 512, 2, "bf16")
    g = to_device(inp)
    y, _ = rg.forward(g["x"], g["conv_w"], g["W_a"], g["b_a"], g["W_x"], g["b_x"], g["Lam"],
                      g["h0"], plan="direct")
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    ws.random_(0, 256)
    a = run_gpu(inp, ct, workspace=ws, y=y)
    ws.random_(0, 256)
    b = run_gpu(inp, ct, workspace=ws, y=y)
    c = run_gpu(inp, ct, y=y)
    for k in NAMES:
        assert np.array_equal(a[k], b[k]) and np.array_equal(a[k], c[k]), k


def test_backward_full_size_rg2b():
    """B=8, T=2048, D=2560, 10 heads of 256, bf16 (the benchmarked layer), every gradient
    against the oracle's full-size backward."""
    inp = make_inputs(WORKLOADS["rg2b"], seed=0)
    ct = make_cotangents(inp, seed=1)
    got = run_gpu(inp, ct)
    ref = run_oracle(inp, ct)
    errs = check(got, ref, TOL["bf16"], names=[n for n in NAMES if n != "dh0"])
    print("full-size backward errors:", errs, flush=True)
