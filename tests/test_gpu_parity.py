"""GPU parity: the HIP path through the C ABI against the fp64 oracle, element by element, on the
same seeded inputs.

Bound (written here, per output tensor y and h_T): err = max_i |y_i - ref_i| / max(|ref_i|, rms(ref))
must stay below 1e-4 for fp32 I/O and 2e-2 for bf16 I/O (fp32 state). The rms floor keeps the
thousands of near-zero states from failing on fp32 rounding alone; a mistake in the method moves
the error by orders of magnitude, not by a factor of two.
Exact cases (bit for bit): the closed recurrence gate (y == h0), head isolation, batch
independence, causality, run-to-run determinism and the conv-state shift of the decode step.
"""
import numpy as np
import pytest
import torch

import gated_linear_recurrence_conv1d_amd as rg
import oracle
from workloads import WORKLOADS, make_inputs, to_device

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def err(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    floor = max(float(np.sqrt(np.mean(ref ** 2))), 1e-30)
    return float(np.max(np.abs(y - ref) / np.maximum(np.abs(ref), floor)))


def host(t):
    return t.float().cpu().numpy()


def gpu_forward(g, plan="auto", chunk_len=0, h0=True):
    y, hT = rg.forward(g["x"], g["conv_w"], g["W_a"], g["b_a"], g["W_x"], g["b_x"], g["Lam"],
                       g["h0"] if h0 else None, plan=plan, chunk_len=chunk_len)
    torch.cuda.synchronize()
    return y, hT


def oracle_forward(inp, h0=True):
    return oracle.forward(inp["x"], inp["conv_w"], inp["W_a"], inp["b_a"], inp["W_x"], inp["b_x"],
                          inp["Lam"], inp["h0"] if h0 else None)


def with_h0(inp, var=0.1, seed=123):
    rng = np.random.default_rng(seed)
    inp = dict(inp)
    inp["h0"] = (rng.standard_normal((inp["B"], inp["D"])) * np.sqrt(var)).astype(np.float32)
    return inp


def case(dtype, B, T, D, H, seed=0, bias=0.25, h0=True, ac=None):
    w = WORKLOADS["tiny"] if dtype == "f32" else WORKLOADS["rg2b"]
    if ac is not None:
        import dataclasses
        w = dataclasses.replace(w, ac_lo=ac[0], ac_hi=ac[1])
    inp = make_inputs(w, seed=seed, B=B, T=T, D=D, H=H, bias_var=bias)
    if h0:
        inp = with_h0(inp)
    return inp


# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,D,H", [("bf16", 512, 2), ("bf16", 256, 2), ("bf16", 256, 4),
                                       ("bf16", 128, 4), ("bf16", 96, 2), ("f32", 256, 16),
                                       ("f32", 96, 2),
                                       ("f32", 512, 2),    # Dh 256: two full output blocks
                                       ("f32", 400, 2),    # Dh 200: second block partial
                                       ("bf16", 264, 2),   # Dh 132: runs of 4 k, partial block
                                       ("f32", 90, 2)])    # Dh 45: the per-output kernel
def test_gate_preacts_match_oracle(dtype, D, H):
    """The gate projection alone (MFMA for bf16 with Dh in {32, 64, 128, 256}, register-tiled
    vector-ALU FMAs for other Dh % 4 == 0 in blocks of 128 outputs, per-output FMAs otherwise)
    against the oracle's pre-activations; 150 rows = two full 64-row tiles and a ragged tail."""
    inp = case(dtype, 2, 150, D, H)
    g = to_device(inp)
    pre = rg.pre_buffer(g["x"])
    rg.rglru_gate_preacts(g["x"], g["conv_w"], g["W_a"], g["b_a"], g["W_x"], g["b_x"], pre)
    torch.cuda.synchronize()
    if dtype == "bf16":
        pair = pre.cpu().numpy().view(np.uint32)
        pa = (pair & 0xFFFF).astype(np.uint16).view(np.float16).astype(np.float64)
        px = (pair >> 16).astype(np.uint16).view(np.float16).astype(np.float64)
        tol = TOL["bf16"]
    else:
        p = pre.cpu().numpy().astype(np.float64)
        pa, px = p[..., 0], p[..., 1]
        tol = 1e-5
    ra, rx = oracle.preacts(inp["x"], inp["conv_w"], inp["W_a"], inp["b_a"], inp["W_x"],
                            inp["b_x"])
    assert err(pa, ra) < tol and err(px, rx) < tol, (err(pa, ra), err(px, rx))


@pytest.mark.parametrize("plan,chunk", [("auto", 0), ("direct", 0), ("chunked", 16),
                                        ("chunked", 37), ("chunked", 100)])
def test_tiny_fp32_config(plan, chunk):
    """B=1, T=256, D=256, 16 heads of 16, fp32 I/O, h0 = 0, seed 0: the CPU-checkable config."""
    inp = make_inputs(WORKLOADS["tiny"], seed=0)
    g = to_device(inp)
    y, hT = gpu_forward(g, plan, chunk)
    yr, hr = oracle_forward(inp)
    assert err(host(y), yr) < TOL["f32"]
    assert err(host(hT), hr) < TOL["f32"]


@pytest.mark.parametrize("dtype,B,T,D,H,plan,chunk", [
    ("bf16", 2, 300, 512, 2, "direct", 0),
    ("bf16", 2, 300, 512, 2, "chunked", 64),   # the one-pass chunked scan: Dh = 256, ragged
    ("bf16", 3, 129, 256, 4, "chunked", 64),   # one-pass, Dh = 64, one row in the last tile
    ("bf16", 2, 150, 512, 4, "chunked", 64),   # one-pass, Dh = 128
    ("bf16", 1, 640, 64, 2, "chunked", 64),    # one-pass, Dh = 32, exact multiple of the tile
    ("bf16", 4, 63, 512, 2, "chunked", 64),    # L = T < 64: the three passes
    ("bf16", 2, 300, 512, 2, "fused", 0),
    ("bf16", 3, 129, 256, 4, "fused", 0),       # Dh = 64, ragged last tile
    ("bf16", 2, 150, 512, 4, "fused", 0),       # Dh = 128, ragged last tile
    ("bf16", 2, 1000, 256, 2, "fused", 0),      # Dh = 128, 16 tiles per sequence
    ("bf16", 1, 640, 64, 2, "fused", 0),        # Dh = 32, exact multiple of the tile
    ("bf16", 4, 63, 512, 2, "fused", 0),        # a single partial tile
    ("bf16", 1, 1, 256, 1, "fused", 0),
    ("bf16", 3, 129, 256, 4, "chunked", 50),
    ("bf16", 1, 200, 128, 4, "auto", 0),
    ("bf16", 2, 77, 96, 2, "auto", 0),          # Dh = 48: vector-ALU gates with bf16 I/O
    ("bf16", 1, 1, 512, 2, "auto", 0),
    ("bf16", 1, 2, 512, 2, "chunked", 1),
    ("bf16", 2, 3, 256, 1, "direct", 0),        # T < conv width; Dh = 256, one head
    ("bf16", 1, 65, 64, 2, "chunked", 16),
    ("f32", 2, 300, 256, 8, "direct", 0),
    ("f32", 2, 300, 256, 8, "chunked", 23),
    ("f32", 1, 5, 48, 3, "auto", 0),
])
def test_forward_small_shapes(dtype, B, T, D, H, plan, chunk):
    """Several tiles, ragged tails, T shorter than the conv, single-step chunks, nonzero biases
    and h0; both scan plans."""
    inp = case(dtype, B, T, D, H, seed=B * 1000 + T)
    g = to_device(inp)
    y, hT = gpu_forward(g, plan, chunk)
    yr, hr = oracle_forward(inp)
    assert err(host(y), yr) < TOL[dtype], err(host(y), yr)
    assert err(host(hT), hr) < TOL[dtype], err(host(hT), hr)


@pytest.mark.parametrize("dtype,plan,chunk", [("bf16", "direct", 0), ("bf16", "chunked", 16),
                                              ("bf16", "fused", 0), ("f32", "direct", 0),
                                              ("f32", "chunked", 16)])
def test_closed_gate_is_bit_exact(dtype, plan, chunk):
    """r = 0 (W_a = 0, b_a = -1e4): a = 1, the normaliser is 0, and the state must be carried
    unchanged bit for bit: y == round(h0), h_T == h0."""
    inp = case(dtype, 2, 90, 512 if dtype == "bf16" else 64, 2)
    inp["W_a"][:] = 0
    inp["b_a"][:] = -1e4
    g = to_device(inp)
    y, hT = gpu_forward(g, plan, chunk)
    h0 = torch.from_numpy(inp["h0"]).cuda()
    expect = h0[:, None, :].expand(y.shape).to(y.dtype)
    assert torch.equal(y, expect)
    assert torch.equal(hT, h0)


def test_decay_zero_gives_gated_input():
    """Lambda = -1e4, r = 1/2: a = 0 and y = sigma(px) * conv(x), whatever h0 is."""
    inp = case("bf16", 2, 130, 512, 2)
    inp["W_a"][:] = 0
    inp["b_a"][:] = 0
    inp["Lam"][:] = -1e4
    g = to_device(inp)
    y, hT = gpu_forward(g)
    yr, hr = oracle_forward(inp)
    assert err(host(y), yr) < TOL["bf16"]


def test_long_decay_range_small():
    """sigma(Lambda)^8 in [0.99, 0.9999] with a small recurrence gate: 1 - a^2 down to ~1e-6,
    where a literal fp32 1 - a*a would be off by ~1e-2; fp32 I/O must still hold 1e-4."""
    inp = case("f32", 2, 400, 64, 2, bias=0.0, ac=(0.99, 0.9999))
    inp["b_a"][:] = -4.0
    g = to_device(inp)
    for plan, chunk in (("direct", 0), ("chunked", 33)):
        y, hT = gpu_forward(g, plan, chunk)
        yr, hr = oracle_forward(inp)
        assert err(host(y), yr) < TOL["f32"], (plan, err(host(y), yr))


def perturbed_runs(g, plan, chunk):
    """y for: the inputs (4 runs), head 1 changed, batch 1 changed, x at t = 101 changed."""
    runs = [gpu_forward(g, plan, chunk)[0] for _ in range(4)]
    g2 = dict(g)
    g2["x"] = g["x"].clone()
    g2["x"][:, :, 256:] = g2["x"][:, :, 256:] * -1.5 + 0.25
    g3 = dict(g)
    g3["x"] = g["x"].clone()
    g3["x"][1] = g3["x"][1].flip(0)
    g4 = dict(g)
    g4["x"] = g["x"].clone()
    g4["x"][:, 101] += 3.0
    return runs, gpu_forward(g2, plan, chunk)[0], gpu_forward(g3, plan, chunk)[0], \
        gpu_forward(g4, plan, chunk)[0]


@pytest.mark.parametrize("plan,chunk", [("chunked", 48), ("direct", 0)])
def test_invariants_bit_exact(plan, chunk):
    """Split plans: determinism, head isolation, batch independence and causality, bit for bit."""
    g = to_device(case("bf16", 3, 200, 512, 2))
    runs, yh, yb, yc = perturbed_runs(g, plan, chunk)
    y = runs[0]
    assert all(torch.equal(y, r) for r in runs[1:])
    assert torch.equal(y[..., :256], yh[..., :256])
    assert torch.equal(y[0], yb[0]) and torch.equal(y[2], yb[2])
    assert torch.equal(y[:, :101], yc[:, :101]) and not torch.equal(y[:, 101], yc[:, 101])


def test_invariants_fused_to_rounding():
    """The fused plan links 64-step tiles by a decoupled look-back whose association order
    depends on timing, so its results are reproducible to fp32 rounding of the carried state,
    not bit for bit. The same invariants must hold to within one bf16 rounding of y, with
    almost every element identical; the first tile of each sequence has no carry and stays
    bit-exact."""
    g = to_device(case("bf16", 3, 200, 512, 2))
    runs, yh, yb, yc = perturbed_runs(g, "fused", 0)
    y = host(runs[0])

    def close(a, b):
        a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
        same = np.mean(a == b)
        return err(a, b) < 1e-2 and same > 0.98

    assert all(close(y, host(r)) for r in runs[1:])
    assert all(torch.equal(runs[0][:, :64], r[:, :64]) for r in runs[1:])
    assert close(y[..., :256], host(yh)[..., :256])
    assert close(y[0], host(yb)[0]) and close(y[2], host(yb)[2])
    assert close(y[:, :101], host(yc)[:, :101]) and not torch.equal(runs[0][:, 101], yc[:, 101])


def test_plans_agree():
    inp = case("bf16", 2, 600, 512, 2)
    g = to_device(inp)
    yd, hd = gpu_forward(g, "direct")
    # chunked with 64-step chunks runs as one pass linked by look-back, like fused: its carried
    # state is reproducible to fp32 rounding, not bitwise like the three-pass form
    for plan, L in (("chunked", 16), ("chunked", 100), ("chunked", 599), ("chunked", 64),
                    ("fused", 0)):
        yc, hc = gpu_forward(g, plan, L)
        assert err(host(yc), host(yd)) < 1e-2
        assert err(host(hc), host(hd)) < (1e-4 if plan == "chunked" and L != 64 else 1e-2)


def test_fused_ignores_workspace_contents():
    """The fused plan clears its look-back words on every call, so neither garbage nor the words
    of earlier calls (of other shapes, on the same buffer) can leak into a result."""
    shapes = [(2, 300, 512, 2), (1, 130, 256, 1), (3, 200, 512, 2)]
    cases = [case("bf16", *s, seed=5 + i) for i, s in enumerate(shapes)]
    need = max(rg.rglru_forward_workspace_size(*s, "bf16") for s in shapes)
    gen = torch.Generator(device="cuda").manual_seed(7)
    ws = torch.randint(0, 256, (need,), dtype=torch.uint8, device="cuda", generator=gen)
    refs = [oracle_forward(c) for c in cases]
    for rep in range(2):
        for c, (y_ref, h_ref), s in zip(cases, refs, shapes):
            g = to_device(c)
            y = torch.empty_like(g["x"])
            hT = torch.empty((s[0], s[2]), dtype=torch.float32, device="cuda")
            rg.rglru_forward_planned(g["x"], g["conv_w"], g["W_a"], g["b_a"], g["W_x"], g["b_x"],
                                     g["Lam"], g["h0"], y, hT, ws, "fused", 0)
            torch.cuda.synchronize()
            assert err(host(y), y_ref) < TOL["bf16"], (rep, s)
            assert err(host(hT), h_ref) < TOL["bf16"], (rep, s)
        # the words the calls left behind become garbage of another kind for the next round
        ws[: need // 2] = torch.randint(0, 256, (need // 2,), dtype=torch.uint8, device="cuda",
                                        generator=gen)


def test_workspace_too_small_is_reported():
    inp = case("bf16", 1, 64, 512, 2)
    g = to_device(inp)
    y = torch.empty_like(g["x"])
    ws = torch.empty(100, dtype=torch.uint8, device="cuda")
    with pytest.raises(rg.RglruError) as e:
        rg.rglru_forward(g["x"], g["conv_w"], g["W_a"], g["b_a"], g["W_x"], g["b_x"], g["Lam"],
                         None, y, None, ws)
    assert e.value.status == rg.RGLRU_ERR_WORKSPACE


# ---------------------------------------------------------------------------------------------
def decode_inputs(N, T, D, H, seed=0):
    inp = make_inputs(WORKLOADS["decode"], seed=seed, B=N, T=T, D=D, H=H, bias_var=0.25)
    return inp, to_device(inp)


@pytest.mark.parametrize("N,D,H", [(70, 512, 2), (100, 512, 4), (5, 256, 4), (3, 96, 2),
                                   (64, 128, 4)])
def test_decode_steps_match_oracle(N, D, H):
    """Several in-place steps: y_t and h within the bf16 bound, conv_state bit-exact."""
    inp, g = decode_inputs(N, 5, D, H)
    cs, h = g["conv_state"].clone(), g["h0"].clone()
    cs_r, h_r = inp["conv_state"], inp["h0"]
    for t in range(5):
        yt = rg.decode_step(g["x"][t], cs, h, g["conv_w"], g["W_a"], g["b_a"], g["W_x"],
                            g["b_x"], g["Lam"])
        torch.cuda.synchronize()
        yr, cs_r, h_r = oracle.decode_step(inp["x"][t], cs_r, h_r, inp["conv_w"], inp["W_a"],
                                           inp["b_a"], inp["W_x"], inp["b_x"], inp["Lam"])
        assert err(host(yt), yr) < TOL["bf16"]
        assert err(host(h), h_r) < TOL["bf16"]
        assert np.array_equal(host(cs), cs_r)


def test_decode_fp32_and_resume_of_forward():
    """fp32: T decode steps from a zero conv state reproduce the oracle's forward at 1e-4; a GPU
    forward over x[:t1] followed by GPU decode steps resumes the sequence."""
    inp = case("f32", 3, 40, 64, 4)
    g = to_device(inp)
    yr, hr = oracle_forward(inp)
    B, T, D = inp["x"].shape
    cs = torch.zeros((B, 3, D), dtype=torch.float32, device="cuda")
    h = g["h0"].clone()
    for t in range(T):
        yt = rg.decode_step(g["x"][:, t].contiguous(), cs, h, g["conv_w"], g["W_a"], g["b_a"],
                            g["W_x"], g["b_x"], g["Lam"])
        torch.cuda.synchronize()
        assert err(host(yt), yr[:, t]) < TOL["f32"]
    t1 = 17
    g1 = dict(g)
    g1["x"] = g["x"][:, :t1].contiguous()
    _, h1 = gpu_forward(g1)
    cs = rg.prefill_state(g1["x"])  # the prefill -> decode hand-off
    assert torch.equal(cs, g["x"][:, t1 - 3:t1])
    h = h1.clone()
    for t in range(t1, T):
        yt = rg.decode_step(g["x"][:, t].contiguous(), cs, h, g["conv_w"], g["W_a"], g["b_a"],
                            g["W_x"], g["b_x"], g["Lam"])
        torch.cuda.synchronize()
        assert err(host(yt), yr[:, t]) < TOL["f32"]


@pytest.mark.parametrize("dtype,B,T,D,H,t1", [("bf16", 2, 200, 512, 2, 130), ("bf16", 3, 70, 96, 2, 2),
                                             ("bf16", 1, 9, 256, 1, 1), ("f32", 2, 50, 24, 2, 5)])
def test_prefill_then_decode_continues_the_sequence(dtype, B, T, D, H, t1):
    """Forward over x[:, :t1] (the automatic plan: fused for bf16 Dh 256), hand-off with
    rglru_prefill_state (zeros before t = 0 when t1 < 3), then decode steps over x[:, t1:] give
    the oracle's forward over the whole sequence."""
    inp = case(dtype, B, T, D, H, seed=T + t1)
    g = to_device(inp)
    yr, hr = oracle_forward(inp)
    g1 = dict(g)
    g1["x"] = g["x"][:, :t1].contiguous()
    _, h = gpu_forward(g1)
    cs = rg.prefill_state(g1["x"])
    expect = torch.zeros_like(cs)
    k = min(3, t1)
    expect[:, 3 - k:] = g["x"][:, t1 - k:t1]
    assert torch.equal(cs, expect)
    for t in range(t1, T):
        yt = rg.decode_step(g["x"][:, t].contiguous(), cs, h, g["conv_w"], g["W_a"], g["b_a"],
                            g["W_x"], g["b_x"], g["Lam"])
        torch.cuda.synchronize()
        assert err(host(yt), yr[:, t]) < TOL[dtype], t
    assert err(h.cpu().numpy(), hr) < TOL[dtype]


# ---------------------------------------------------------------------------------------------
# Full sizes, in the launch configuration the benchmark times (automatic plan); outputs are
# sampled per (batch, head): a head's channels depend only on that head's inputs, so the oracle
# computes the sampled sub-problems exactly as it would inside the full one.
def sub_problem(inp, b, g):
    Dh = inp["D"] // inp["H"]
    s = slice(g * Dh, (g + 1) * Dh)
    return dict(x=inp["x"][b:b + 1, :, s], conv_w=inp["conv_w"][:, s], W_a=inp["W_a"][g:g + 1],
                b_a=inp["b_a"][s], W_x=inp["W_x"][g:g + 1], b_x=inp["b_x"][s], Lam=inp["Lam"][s],
                h0=None if inp["h0"] is None else inp["h0"][b:b + 1, s])


@pytest.mark.parametrize("name,samples", [("rg2b", [(0, 0), (7, 9), (3, 4)]),
                                          ("rg9b", [(0, 15), (15, 0)]),
                                          ("long", [(0, 3)])])
def test_full_size_sampled(name, samples):
    w = WORKLOADS[name]
    inp = make_inputs(w, seed=0)
    g = to_device(inp)
    y, hT = gpu_forward(g)
    Dh = w.D // w.H
    for b, hd in samples:
        sp = sub_problem(inp, b, hd)
        yr, hr = oracle_forward(sp)
        ys = y[b:b + 1, :, hd * Dh:(hd + 1) * Dh]
        assert err(host(ys), yr) < TOL["bf16"], (name, b, hd, err(host(ys), yr))
        assert err(host(hT[b:b + 1, hd * Dh:(hd + 1) * Dh]), hr) < TOL["bf16"]
    del y, hT, g
    torch.cuda.empty_cache()


def test_full_size_long_plans_agree():
    """The long config (B=1, T=65536): the automatic (fused, 1024 tiles per sequence linked by
    the look-back), chunked and direct plans must agree across all 2560 channels and all 65536
    steps."""
    inp = make_inputs(WORKLOADS["long"], seed=0)
    g = to_device(inp)
    yf, hf = gpu_forward(g)
    yd, hd = gpu_forward(g, "direct")
    yc, hc = gpu_forward(g, "chunked")
    assert err(host(hc), host(hd)) < 1e-3
    assert err(host(hf), host(hd)) < 1e-2
    assert err(host(yc[:, -4096:]), host(yd[:, -4096:])) < 1e-2
    assert err(host(yf), host(yd)) < 2e-2


def test_full_size_decode_256_steps():
    """1024 rows, D = 4096, 16 heads, 256 consecutive in-place steps; four rows are followed by
    the oracle through all 256 steps (rows are independent)."""
    w = WORKLOADS["decode"]
    inp = make_inputs(w, seed=0)
    g = to_device(inp)
    cs, h = g["conv_state"].clone(), g["h0"].clone()
    rows = [0, 1, 511, 1023]
    cs_r, h_r = inp["conv_state"][rows], inp["h0"][rows]
    y_t = torch.empty_like(g["x"][0])
    worst = 0.0
    for t in range(w.T):
        rg.rglru_decode_step(g["x"][t], cs, h, y_t, g["conv_w"], g["W_a"], g["b_a"], g["W_x"],
                             g["b_x"], g["Lam"])
        yr, cs_r, h_r = oracle.decode_step(inp["x"][t][rows], cs_r, h_r, inp["conv_w"],
                                           inp["W_a"], inp["b_a"], inp["W_x"], inp["b_x"],
                                           inp["Lam"])
        if t % 32 == 31 or t == w.T - 1:
            torch.cuda.synchronize()
            worst = max(worst, err(host(y_t[rows]), yr))
    torch.cuda.synchronize()
    assert worst < TOL["bf16"]
    assert err(host(h[rows]), h_r) < TOL["bf16"]
    assert np.array_equal(host(cs[rows]), cs_r)
