"""Host-side checks of the C ABI (no GPU, no kernel launch): the library loads, exports every
entry point include/rglru.h declares, sizes its workspace as documented, picks plans, and rejects
bad arguments with the documented status before any launch."""
import ctypes
import os
import re

import pytest

import gated_linear_recurrence_conv1d_amd as rg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rglru.h")
lib = rg._lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rglru_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 9, names
    for n in names:
        assert hasattr(lib, n), f"librglru.so does not export {n}"


def test_status_strings():
    for code in range(5):
        s = rg.rglru_status_string(code)
        assert isinstance(s, str) and s
    assert rg.rglru_status_string(0) == "ok"
    assert "unknown" in rg.rglru_status_string(99)


def test_workspace_sizes():
    B, T, D, H = 8, 2048, 2560, 10
    tiles = (T // 64) * B * H
    assert rg.rglru_forward_workspace_size(B, T, D, H, "bf16") >= 256 + 2 * tiles * (D // H) * 8
    pre = B * T * D * 4
    nC = (T + 15) // 16
    scan = B * nC * D * 8 + B * nC * D * 4
    assert rg.rglru_scan_workspace_size(B, T, D, H, "bf16") >= scan
    assert rg.rglru_forward_workspace_size(B, T, D, H, "bf16") >= pre + scan
    assert rg.rglru_forward_workspace_size(B, T, D, H, "f32") >= 2 * pre + scan
    assert rg.rglru_forward_workspace_size(B, T, D, 7, "bf16") == 0   # D % H != 0
    assert rg.rglru_forward_workspace_size(0, T, D, H, "bf16") == 0
    assert rg.rglru_forward_workspace_size(1, 1, 1024, 2, "bf16") == 0  # Dh = 512 > 256


def test_auto_plan_choices():
    # bf16 with Dh in {32, 64, 128, 256}: the single-pass fused plan over 64-step tiles
    assert rg.rglru_forward_plan_info(16, 4096, 4096, 16, "bf16") == ("fused", 64)
    assert rg.rglru_forward_plan_info(8, 2048, 2560, 10, "bf16") == ("fused", 64)
    assert rg.rglru_forward_plan_info(1, 65536, 2560, 10, "bf16") == ("fused", 64)
    # otherwise the split plans, chosen by how many channels there are to spread over lanes
    # (direct from B * D >= 128K lanes; chunks of at most 64 steps, shorter while the chunked
    # lanes B * D * n_chunks stay below 512K)
    assert rg.rglru_forward_plan_info(32, 4096, 4800, 100, "bf16") == ("direct", 4096)  # Dh 48
    assert rg.rglru_forward_plan_info(16, 4096, 4800, 100, "bf16") == ("chunked", 64)
    plan, L = rg.rglru_forward_plan_info(8, 2048, 2400, 50, "bf16")
    assert plan == "chunked" and 16 <= L <= 64
    assert (8 * 2400) * ((2048 + L - 1) // L) >= 8 * 65536
    plan, L = rg.rglru_forward_plan_info(1, 256, 256, 16, "f32")
    assert plan == "chunked" and L == 16
    plan, L = rg.rglru_forward_plan_info(1, 4096, 2560, 10, "f32")
    assert plan == "chunked" and 16 <= L < 64 and 2560 * ((4096 + L - 1) // L) >= 8 * 65536
    assert rg.rglru_forward_plan_info(1, 10, 256, 16, "f32") == ("direct", 10)
    assert rg.rglru_forward_plan_info(32, 4096, 4096, 16, "f32") == ("direct", 4096)
    assert rg.rglru_forward_plan_info(16, 4096, 4096, 16, "f32") == ("chunked", 64)


FAKE = 0x10000  # never dereferenced: every call below fails its checks before any launch


def fwd(**kw):
    a = dict(x=FAKE, conv_w=FAKE + 0x1000, W_a=FAKE + 0x2000, b_a=FAKE + 0x3000,
             W_x=FAKE + 0x4000, b_x=FAKE + 0x5000, Lam=FAKE + 0x6000, h0=None,
             y=0x7000000000, h_T=None, B=2, T=64, D=512, H=2, dt=rg.RGLRU_BF16, ws=None,
             wsb=0, stream=None, plan=rg.RGLRU_PLAN_AUTO, chunk=0)
    a.update(kw)
    return lib.rglru_forward_planned(a["x"], a["conv_w"], a["W_a"], a["b_a"], a["W_x"],
                                     a["b_x"], a["Lam"], a["h0"], a["y"], a["h_T"], a["B"],
                                     a["T"], a["D"], a["H"], a["dt"], a["ws"], a["wsb"],
                                     a["stream"], a["plan"], a["chunk"])


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), rg.RGLRU_ERR_INVALID_ARG),
    (dict(y=None), rg.RGLRU_ERR_INVALID_ARG),
    (dict(W_x=None), rg.RGLRU_ERR_INVALID_ARG),
    (dict(Lam=None), rg.RGLRU_ERR_INVALID_ARG),
    (dict(B=0), rg.RGLRU_ERR_INVALID_ARG),
    (dict(T=0), rg.RGLRU_ERR_INVALID_ARG),
    (dict(H=3), rg.RGLRU_ERR_INVALID_ARG),
    (dict(D=1024, H=2), rg.RGLRU_ERR_UNSUPPORTED),    # Dh = 512
    (dict(dt=7), rg.RGLRU_ERR_UNSUPPORTED),
    (dict(x=FAKE + 2), rg.RGLRU_ERR_INVALID_ARG),     # misaligned
    (dict(y=FAKE), rg.RGLRU_ERR_INVALID_ARG),         # y aliases x
    (dict(), rg.RGLRU_ERR_WORKSPACE),                 # no workspace
    (dict(ws=0x9000000000, wsb=100), rg.RGLRU_ERR_WORKSPACE),
    (dict(plan=9), rg.RGLRU_ERR_INVALID_ARG),
    (dict(plan=rg.RGLRU_PLAN_CHUNKED, chunk=-1), rg.RGLRU_ERR_INVALID_ARG),
    (dict(plan=rg.RGLRU_PLAN_FUSED, D=96, H=2), rg.RGLRU_ERR_UNSUPPORTED),   # Dh = 48
    (dict(plan=rg.RGLRU_PLAN_FUSED, dt=rg.RGLRU_F32), rg.RGLRU_ERR_UNSUPPORTED),
    (dict(plan=rg.RGLRU_PLAN_FUSED), rg.RGLRU_ERR_WORKSPACE),
])
def test_forward_argument_checks(kw, status):
    assert fwd(**kw) == status


def test_forward_workspace_overlapping_output_rejected():
    n = rg.rglru_forward_workspace_size(2, 64, 512, 2, "bf16")
    y = 0x7000000000
    assert fwd(ws=y + 256, wsb=n) == rg.RGLRU_ERR_INVALID_ARG


def test_decode_argument_checks():
    def dec(**kw):
        a = dict(x_t=FAKE, cs=FAKE + 0x100000, h=FAKE + 0x200000, y_t=FAKE + 0x300000,
                 conv_w=FAKE + 0x400000, W_a=FAKE + 0x500000, b_a=FAKE + 0x600000,
                 W_x=FAKE + 0x700000, b_x=FAKE + 0x800000, Lam=FAKE + 0x900000, N=4, D=512,
                 H=2, dt=rg.RGLRU_BF16)
        a.update(kw)
        return lib.rglru_decode_step(a["x_t"], a["cs"], a["h"], a["y_t"], a["conv_w"], a["W_a"],
                                     a["b_a"], a["W_x"], a["b_x"], a["Lam"], a["N"], a["D"],
                                     a["H"], a["dt"], None)
    assert dec(N=0) == rg.RGLRU_ERR_INVALID_ARG
    assert dec(h=None) == rg.RGLRU_ERR_INVALID_ARG
    assert dec(y_t=FAKE) == rg.RGLRU_ERR_INVALID_ARG          # y_t aliases x_t
    assert dec(y_t=FAKE + 0x100000 + 2048) == rg.RGLRU_ERR_INVALID_ARG  # inside conv_state
    assert dec(D=1024) == rg.RGLRU_ERR_UNSUPPORTED
    assert dec(cs=FAKE + 0x100004) == rg.RGLRU_ERR_INVALID_ARG  # misaligned
    assert dec(dt=5) == rg.RGLRU_ERR_UNSUPPORTED


def test_local_mqa_argument_checks():
    def mqa(**kw):
        a = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, o=FAKE + 0x300000, B=2, T=64, Hq=2,
                 dh=128, window=16, scale=0.0, dt=rg.RGLRU_BF16)
        a.update(kw)
        return lib.rglru_local_mqa(a["q"], a["k"], a["v"], a["o"], a["B"], a["T"], a["Hq"],
                                   a["dh"], a["window"], a["scale"], a["dt"], None)
    assert mqa(B=0) == rg.RGLRU_ERR_INVALID_ARG
    assert mqa(window=0) == rg.RGLRU_ERR_INVALID_ARG
    assert mqa(v=None) == rg.RGLRU_ERR_INVALID_ARG
    assert mqa(dh=96) == rg.RGLRU_ERR_UNSUPPORTED
    assert mqa(dt=rg.RGLRU_F32) == rg.RGLRU_ERR_UNSUPPORTED
    assert mqa(T=(1 << 21) + 1, dh=256) == rg.RGLRU_ERR_UNSUPPORTED  # k of one sequence > 1 GiB
    assert mqa(k=FAKE + 0x100008) == rg.RGLRU_ERR_INVALID_ARG        # misaligned
    assert mqa(scale=-1.0) == rg.RGLRU_ERR_INVALID_ARG
    assert mqa(scale=float("nan")) == rg.RGLRU_ERR_INVALID_ARG
    assert mqa(o=FAKE + 0x200000 + 4096) == rg.RGLRU_ERR_INVALID_ARG  # o overlaps v
    assert mqa(o=FAKE) == rg.RGLRU_ERR_INVALID_ARG                    # o is q


def test_gate_and_scan_stage_checks():
    assert lib.rglru_gate_preacts(FAKE, FAKE + 0x1000, FAKE + 0x2000, FAKE + 0x3000,
                                  FAKE + 0x4000, FAKE + 0x5000, None, 2, 64, 512, 2,
                                  rg.RGLRU_BF16, None) == rg.RGLRU_ERR_INVALID_ARG
    assert lib.rglru_gate_preacts(FAKE, FAKE + 0x1000, FAKE + 0x2000, FAKE + 0x3000,
                                  FAKE + 0x4000, FAKE + 0x5000, FAKE, 2, 64, 512, 2,
                                  rg.RGLRU_BF16, None) == rg.RGLRU_ERR_INVALID_ARG  # pre aliases x
    # the fused plan has no separate scan stage
    assert lib.rglru_scan_preacts(FAKE, 0x8000000000, FAKE + 0x1000, FAKE + 0x2000, None,
                                  0x7000000000, None, 2, 64, 512, 2, rg.RGLRU_BF16, None, 0,
                                  None, rg.RGLRU_PLAN_FUSED, 0) == rg.RGLRU_ERR_INVALID_ARG
    # chunked scan without workspace
    assert lib.rglru_scan_preacts(FAKE, 0x8000000000, FAKE + 0x1000, FAKE + 0x2000, None,
                                  0x7000000000, None, 2, 64, 512, 2, rg.RGLRU_BF16, None, 0,
                                  None, rg.RGLRU_PLAN_CHUNKED, 16) == rg.RGLRU_ERR_WORKSPACE


def bwd(**kw):
    """rglru_backward with fake, well separated device addresses (B=2, T=64, D=512, H=2)."""
    base = 0x100000000
    names = ["x", "conv_w", "W_a", "b_a", "W_x", "b_x", "Lam", "h0", "y", "dy", "dh_T", "dx",
             "dconv_w", "dW_a", "db_a", "dW_x", "db_x", "dLam", "dh0"]
    a = {n: base + k * 0x1000000 for k, n in enumerate(names)}
    a.update(B=2, T=64, D=512, H=2, dt=rg.RGLRU_BF16, ws=base + 40 * 0x1000000, wsb=1 << 40)
    a.update(kw)
    return lib.rglru_backward(*[a[n] for n in names], a["B"], a["T"], a["D"], a["H"], a["dt"],
                              a["ws"], a["wsb"], None)


def test_backward_workspace_size():
    B, T, D, H = 8, 2048, 2560, 10
    n = B * T * D
    # gate-gradient pairs (two fp16 for bf16 I/O) and conv-output gradients (fp16 for bf16 I/O,
    # fp32 for fp32); the unfused plan adds the pre-activation pairs
    assert rg.rglru_backward_workspace_size(B, T, D, H, "bf16") >= n * (4 + 2)
    assert rg.rglru_backward_workspace_size(B, T, D, H, "f32") >= n * (8 + 8 + 4)
    assert rg.rglru_backward_workspace_size(B, T, D, 7, "bf16") == 0
    assert rg.rglru_backward_workspace_size(1, 1, 1024, 2, "bf16") == 0


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), rg.RGLRU_ERR_INVALID_ARG),
    (dict(y=None), rg.RGLRU_ERR_INVALID_ARG),
    (dict(dy=None), rg.RGLRU_ERR_INVALID_ARG),
    (dict(dW_x=None), rg.RGLRU_ERR_INVALID_ARG),
    (dict(dLam=None), rg.RGLRU_ERR_INVALID_ARG),
    (dict(T=0), rg.RGLRU_ERR_INVALID_ARG),
    (dict(H=3), rg.RGLRU_ERR_INVALID_ARG),
    (dict(D=1024, H=2), rg.RGLRU_ERR_UNSUPPORTED),
    (dict(dt=9), rg.RGLRU_ERR_UNSUPPORTED),
    (dict(dx=0x100000000 + 8), rg.RGLRU_ERR_INVALID_ARG),        # misaligned
    (dict(dx=0x100000000 + 9 * 0x1000000), rg.RGLRU_ERR_INVALID_ARG),   # dx aliases dy
    (dict(db_a=0x100000000 + 13 * 0x1000000 + 64), rg.RGLRU_ERR_INVALID_ARG),  # inside dW_a
    (dict(dh0=0x100000000 + 40 * 0x1000000), rg.RGLRU_ERR_INVALID_ARG),  # in the workspace
    (dict(ws=None), rg.RGLRU_ERR_WORKSPACE),
    (dict(wsb=1000), rg.RGLRU_ERR_WORKSPACE),
])
def test_backward_argument_checks(kw, status):
    assert bwd(**kw) == status


def test_prefill_state_argument_checks():
    x, cs = 0x100000000, 0x200000000
    ok_shape = (2, 64, 512, rg.RGLRU_BF16)
    assert lib.rglru_prefill_state(None, cs, *ok_shape, None) == rg.RGLRU_ERR_INVALID_ARG
    assert lib.rglru_prefill_state(x, None, *ok_shape, None) == rg.RGLRU_ERR_INVALID_ARG
    assert lib.rglru_prefill_state(x, x + 4096, *ok_shape, None) == rg.RGLRU_ERR_INVALID_ARG  # overlap
    assert lib.rglru_prefill_state(x + 8, cs, *ok_shape, None) == rg.RGLRU_ERR_INVALID_ARG    # align
    assert lib.rglru_prefill_state(x, cs, 0, 64, 512, rg.RGLRU_BF16, None) == rg.RGLRU_ERR_INVALID_ARG
    assert lib.rglru_prefill_state(x, cs, 2, 64, 512, 9, None) == rg.RGLRU_ERR_UNSUPPORTED


def test_planned_workspace_sizes():
    B, T, D, H = 8, 2048, 2560, 10
    ctrl = 256
    pre = B * T * D * 4
    fused = rg.rglru_forward_workspace_size_planned(B, T, D, H, "bf16", "fused", 0)
    assert fused >= ctrl + (T // 64) * B * D * 8
    assert rg.rglru_forward_workspace_size_planned(B, T, D, H, "bf16", "auto", 0) == fused
    direct = rg.rglru_forward_workspace_size_planned(B, T, D, H, "bf16", "direct", 0)
    assert direct >= ctrl + pre
    for L in (1, 7, 64, 5000):
        nC = (T + min(L, T) - 1) // min(L, T)
        got = rg.rglru_forward_workspace_size_planned(B, T, D, H, "bf16", "chunked", L)
        assert got >= direct + B * nC * D * 12, L
    # explicit chunks shorter than 16 steps need more than the plan-independent query gives
    assert rg.rglru_forward_workspace_size_planned(B, T, D, H, "bf16", "chunked", 1) > \
        rg.rglru_forward_workspace_size(B, T, D, H, "bf16")
    # the plan-independent size covers every plan with chunks of >= 16 steps
    for plan, L in (("fused", 0), ("direct", 0), ("chunked", 16), ("chunked", 0)):
        assert rg.rglru_forward_workspace_size_planned(B, T, D, H, "bf16", plan, L) <= \
            rg.rglru_forward_workspace_size(B, T, D, H, "bf16")
    # invalid: unsupported fused shape, negative chunk, bad shape
    assert rg.rglru_forward_workspace_size_planned(1, 64, 96, 2, "bf16", "fused", 0) == 0
    assert rg.rglru_forward_workspace_size_planned(1, 64, 256, 1, "f32", "fused", 0) == 0
    assert rg.rglru_forward_workspace_size_planned(1, 64, 256, 1, "bf16", "chunked", -1) == 0
    assert rg.rglru_forward_workspace_size_planned(1, 64, 256, 3, "bf16", "direct", 0) == 0


def test_lookback_failures_argument_checks():
    n = ctypes.c_uint(7)
    assert lib.rglru_lookback_failures(None, 1 << 20, ctypes.byref(n), None) == \
        rg.RGLRU_ERR_INVALID_ARG
    assert lib.rglru_lookback_failures(FAKE, 255, ctypes.byref(n), None) == \
        rg.RGLRU_ERR_INVALID_ARG
    assert lib.rglru_lookback_failures(FAKE, 256, None, None) == rg.RGLRU_ERR_INVALID_ARG
    assert lib.rglru_lookback_failures(FAKE + 8, 256, ctypes.byref(n), None) == \
        rg.RGLRU_ERR_INVALID_ARG
    assert n.value == 7


def test_binding_checks_every_tensor_size():
    """The binding checks each tensor's shape against (B, T, D, H) before any call, so that a
    wrong-sized buffer never reaches the device (host tensors: nothing is launched)."""
    import torch
    B, T, D, H = 2, 5, 64, 2
    Dh = D // H
    bf, f32 = torch.bfloat16, torch.float32
    x = torch.zeros(B, T, D, dtype=bf)
    p = dict(conv_w=torch.zeros(4, D, dtype=bf), W_a=torch.zeros(H, Dh, Dh, dtype=bf),
             b_a=torch.zeros(D), W_x=torch.zeros(H, Dh, Dh, dtype=bf), b_x=torch.zeros(D),
             Lambda=torch.zeros(D))
    good = dict(h0=torch.zeros(B, D), y=torch.zeros(B, T, D, dtype=bf), h_T=torch.zeros(B, D))
    bad = {"conv_w": torch.zeros(3, D, dtype=bf), "W_x": torch.zeros(H, Dh, Dh + 1, dtype=bf),
           "b_a": torch.zeros(D - 1), "Lambda": torch.zeros(D + 1), "h0": torch.zeros(B + 1, D),
           "y": torch.zeros(B, T - 1, D, dtype=bf), "h_T": torch.zeros(B, D // 2)}
    ws = torch.zeros(1 << 16, dtype=torch.uint8)
    for name, t in bad.items():
        args = dict(p, **good)
        args[name] = t
        with pytest.raises(ValueError, match=name):
            rg.rglru_forward(x, args["conv_w"], args["W_a"], args["b_a"], args["W_x"],
                             args["b_x"], args["Lambda"], args["h0"], args["y"], args["h_T"], ws)
    with pytest.raises(ValueError, match="pre"):
        rg.rglru_gate_preacts(x, p["conv_w"], p["W_a"], p["b_a"], p["W_x"], p["b_x"],
                              torch.zeros(B, T, D - 2, dtype=torch.int32))
    with pytest.raises(ValueError, match="pre"):
        rg.rglru_scan_preacts(x, torch.zeros(B, T, D, 2), p["conv_w"], p["Lambda"], None,
                              good["y"], None, H)
    N = 3
    with pytest.raises(ValueError, match="conv_state"):
        rg.rglru_decode_step(torch.zeros(N, D, dtype=bf), torch.zeros(N, 2, D, dtype=bf),
                             torch.zeros(N, D), torch.zeros(N, D, dtype=bf), **p)
    with pytest.raises(ValueError, match="h"):
        rg.rglru_decode_step(torch.zeros(N, D, dtype=bf), torch.zeros(N, 3, D, dtype=bf),
                             torch.zeros(N + 1, D), torch.zeros(N, D, dtype=bf), **p)
    with pytest.raises(ValueError, match="conv_state"):
        rg.rglru_prefill_state(x, torch.zeros(B, 3, D + 1, dtype=bf))
    with pytest.raises(ValueError, match="k"):
        rg.rglru_local_mqa(torch.zeros(B, T, 2, 64, dtype=bf), torch.zeros(B, T + 1, 64, dtype=bf),
                           torch.zeros(B, T, 64, dtype=bf), torch.zeros(B, T, 2, 64, dtype=bf), 4)
    grads = dict(dx=torch.zeros(B, T, D, dtype=bf), dconv_w=torch.zeros(4, D),
                 dW_a=torch.zeros(H, Dh, Dh), db_a=torch.zeros(D), dW_x=torch.zeros(H, Dh, Dh),
                 db_x=torch.zeros(D), dLambda=torch.zeros(D), dh0=torch.zeros(B, D))
    for name in grads:
        g = dict(grads)
        g[name] = torch.zeros(1)
        with pytest.raises(ValueError, match=name):
            rg.rglru_backward(x, p["conv_w"], p["W_a"], p["b_a"], p["W_x"], p["b_x"], p["Lambda"],
                              None, good["y"], good["y"], None, g["dx"], g["dconv_w"], g["dW_a"],
                              g["db_a"], g["dW_x"], g["db_x"], g["dLambda"], g["dh0"], ws)
