"""The local MQA kernel rounds its probabilities P to bf16 alone in query blocks whose rows all see
at least 256 keys, and splits P into bf16 hi + lo elsewhere. This fp64 emulation of the rounding
(no GPU) pins that choice against the GPU tests' error bound: bf16 P on rows with 256 keys or more
stays inside it, bf16 P on every row does not (rows with few keys whose output cancels). The case
is the GPU test's B1 T1100 Hq2 dh256 W1024 one, with its seed."""
import numpy as np
import pytest

from workloads import make_attention_inputs, round_to_dtype

BOUND = 2e-2  # the bound of tests/test_gpu_mqa.py


def bf16(a):
    return round_to_dtype(np.asarray(a, np.float32), "bf16").astype(np.float64)


def emulate(n_min, T=1100, Hq=2, dh=256, W=1024, seed=1100 + 1024):
    """Worst element error (metric of the GPU tests) with P in bf16 on rows of >= n_min keys and
    exact elsewhere; the output rounded to bf16 as the kernel stores it."""
    inp = make_attention_inputs(1, T, Hq, dh, seed=seed)
    q, k, v = (inp[n][0].astype(np.float64) for n in ("q", "k", "v"))
    ref = np.zeros((T, Hq, dh))
    got = np.zeros((T, Hq, dh))
    for h in range(Hq):
        S = q[:, h, :] @ k.T / np.sqrt(dh)
        for t in range(T):
            lo = max(0, t - W + 1)
            s = S[t, lo:t + 1]
            p = np.exp(s - s.max())
            l = p.sum()
            ref[t, h] = p @ v[lo:t + 1] / l
            pp = bf16(p) if t + 1 >= n_min else p
            got[t, h] = pp @ v[lo:t + 1] / l
    floor = np.sqrt(np.mean(ref ** 2))
    return float(np.max(np.abs(bf16(got) - ref) / np.maximum(np.abs(ref), floor)))


def test_bf16_p_beyond_256_keys_is_inside_the_bound():
    assert emulate(256) < 0.6 * BOUND


def test_bf16_p_on_every_row_is_not():
    assert emulate(1) > BOUND
