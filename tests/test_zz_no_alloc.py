"""The allocation-free forward (rglru_forward_noalloc) through the C ABI: its output against
rglru_forward's on the same inputs, on two calls in a row with the second smaller, and the size
limit rejected before any launch.

Bound: the parity tests' err < 2e-2 (bf16) / 1e-4 (fp32) against rglru_forward's output; the
fused plan links tiles by a look-back whose association order depends on timing, so its results
agree to fp32 rounding of the carried state; the split plans agree bit for bit.
"""
import numpy as np
import pytest
import torch

import gated_linear_recurrence_conv1d_amd as rg
from workloads import WORKLOADS, make_inputs, to_device

pytestmark = pytest.mark.gpu


def err(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    floor = max(float(np.sqrt(np.mean(ref ** 2))), 1e-30)
    return float(np.max(np.abs(y - ref) / np.maximum(np.abs(ref), floor)))


def both(g, h0=True):
    x = g["x"]
    B, T, D = x.shape
    args = (x, g["conv_w"], g["W_a"], g["b_a"], g["W_x"], g["b_x"], g["Lam"],
            g["h0"] if h0 else None)
    y1, h1 = torch.empty_like(x), torch.empty((B, D), dtype=torch.float32, device="cuda")
    y2, h2 = torch.empty_like(x), torch.empty((B, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(rg.rglru_forward_workspace_size(B, T, D, g["W_a"].shape[0], x.dtype),
                     dtype=torch.uint8, device="cuda")
    rg.rglru_forward(*args, y1, h1, ws)
    rg.rglru_forward_noalloc(*args, y2, h2)
    torch.cuda.synchronize()
    return (y1.float().cpu().numpy(), h1.cpu().numpy()), (y2.float().cpu().numpy(),
                                                           h2.cpu().numpy())


@pytest.mark.parametrize("dtype,first,second", [
    ("bf16", (8, 2048, 2560, 10), (2, 300, 512, 2)),    # fused plan: the benchmark layer, then small
    ("f32", (2, 700, 256, 8), (1, 90, 64, 2)),          # split plan (chunked / direct)
])
def test_noalloc_matches_forward_twice(dtype, first, second):
    w = WORKLOADS["rg2b"] if dtype == "bf16" else WORKLOADS["tiny"]
    tol = 2e-2 if dtype == "bf16" else 1e-4
    for i, (B, T, D, H) in enumerate((first, second)):
        inp = make_inputs(w, seed=30 + i, B=B, T=T, D=D, H=H, bias_var=0.25)
        rng = np.random.default_rng(40 + i)
        inp["h0"] = (rng.standard_normal((B, D)) * np.sqrt(0.1)).astype(np.float32)
        g = to_device(inp)
        (ya, ha), (yb, hb) = both(g)
        assert err(yb, ya) < tol and err(hb, ha) < tol, (i, err(yb, ya), err(hb, ha))
        if dtype == "bf16":
            assert np.mean(ya == yb) > 0.98
        else:
            assert np.array_equal(ya, yb) and np.array_equal(ha, hb)


def test_noalloc_rejects_shapes_beyond_its_array():
    cap = rg.rglru_forward_noalloc_max_bytes()
    assert cap == 72 << 20
    # B * T * D / 4 bytes of look-back words exceed the array: refused before any launch
    B, T, D, H = 64, 8192, 2560, 10
    assert rg.rglru_forward_workspace_size_planned(B, T, D, H, "bf16") > cap
    x = torch.empty((B, T, D), dtype=torch.bfloat16, device="cuda")
    inp = make_inputs(WORKLOADS["rg2b"], seed=0, B=1, T=1, D=D, H=H)
    g = to_device(inp)
    y = torch.empty_like(x)
    with pytest.raises(rg.RglruError) as e:
        rg.rglru_forward_noalloc(x, g["conv_w"], g["W_a"], g["b_a"], g["W_x"], g["b_x"], g["Lam"],
                                 None, y, None)
    assert e.value.status == rg.RGLRU_ERR_UNSUPPORTED
