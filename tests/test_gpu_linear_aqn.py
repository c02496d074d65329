"""GPU parity of the projection of the noisy RMSNorm (fp4w_linear_aqn) against the
binary64 oracle (oracle.linear_aqn: the norm, then the linear with its LoRA
branch, no rounding between).

Bound, per output (m, n), with x~ the oracle's normalized row and w the effective
weight row deq(W)[n] + (B A)[n]:
    |y - y64| <= 2e-3 ||x~_m|| ||w_n|| + 2^-8 sum_k |x~_mk w_nk|
The first term is the linear's own bound on exact bf16 inputs; the second covers
the one rounding of x~ to bf16 (2^-9 of each term), which both routes take (the
fused kernel rounds x gamma (1 + sigma noise) and applies the row factor to the
fp32 sums; the two-launch route rounds x~ itself), and the fp32 sum of squares
behind the row factor (under 2^-12 relative for k <= 2^12 positive terms).
Cases: the fused routes -- the block-scaled decode kernel (m <= 2, one K slice)
and the x-in-registers decode kernel (m = 5 .. 16, one K span) -- on the
Qwen-2.5-7B 3584-wide inputs, both formats, with and without LoRA, ragged n, k
and rank; the two-launch route (K splits: 3584 x 18944 at m = 1 and m = 8, and
m = 40 on the GEMM); outputs pre-filled with NaN; and the fused result against
the two-launch result on the same inputs."""
import numpy as np
import pytest
import torch

import oracle as O
from mxfp4_bit_weight_amd import workloads as W
from tests.gpu_util import DEV, Guarded, bf16_dev, bits_host, f32_dev, f64_of_bf16, qweight_dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp4w():
    from mxfp4_bit_weight_amd import fp4w as F
    return F


def _case(seed, fmt, m, n, k, r):
    w = W.weights("outlier" if fmt == 0 else "student_t", seed, W.TID_W, (n, k))
    x = W.normal_bf16(seed, W.TID_X, (m, k), 3.0)
    rng = np.random.default_rng(seed)
    gamma = W.to_bf16_bits(1.0 + 0.2 * rng.standard_normal(k))
    noise = rng.standard_normal(k).astype(np.float32)
    a = W.normal_bf16(seed, W.TID_A, (r, k), 0.05) if r else None
    b = W.normal_bf16(seed, W.TID_B, (n, r), 0.05) if r else None
    codes, scales, st = O.quantize(fmt, w)
    return x, gamma, noise, codes, scales, st, a, b


def _check(fmt, got, x, gamma, noise, sigma, eps, codes, scales, st, a, b, what):
    y64 = O.linear_aqn(fmt, x, gamma, noise, sigma, eps, codes, scales, st, a, b)
    xt = O.aqn_rmsnorm(x, gamma, noise, sigma, eps)
    weff = O.dequantize(fmt, codes, scales, st, "f64")
    if a is not None:
        weff = weff + f64_of_bf16(b) @ f64_of_bf16(a)
    xn = np.linalg.norm(xt, axis=1)[:, None]
    wn = np.linalg.norm(weff, axis=1)[None, :]
    lim = 2e-3 * xn * wn + 2.0 ** -8 * (np.abs(xt) @ np.abs(weff).T)
    err = np.abs(got - y64)
    bad = ~(err <= lim)
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outputs outside the bound, worst "
                           f"{float(np.max(np.where(np.isfinite(err), err / lim, np.inf))):.2f}x")


def _run(fp4w, fmt, x, gamma, noise, sigma, eps, codes, scales, st, a, b):
    q = qweight_dev(fp4w, fmt, codes, scales, st)
    m, n = x.shape[0], codes.shape[0]
    g = Guarded((m, n), torch.bfloat16, float("nan"))
    out = g.t
    fp4w.linear_aqn(bf16_dev(x), bf16_dev(gamma), f32_dev(noise), sigma, q,
                    bf16_dev(a) if a is not None else None, bf16_dev(b) if b is not None else None, eps=eps, out=out)
    g.check(f"linear aqn m={m} n={n}")
    return f64_of_bf16(bits_host(out)), q


FUSED = [(1, 3584, 3584, 0), (1, 3584, 3584, 16), (2, 3584, 3584, 16), (1, 18944, 3584, 16), (2, 18944, 3584, 0),
         (1, 200, 96, 5), (2, 264, 544, 17), (1, 1032, 4128, 64),
         (8, 3584, 3584, 16), (8, 18944, 3584, 16), (16, 4608, 3584, 0), (5, 264, 544, 17), (5, 1032, 1056, 16),
         (12, 200, 4096, 64),
         (16, 18944, 3584, 64),     # the gain's LDS leaves no room for staged scales: per-lane scale loads
         (6, 72, 64, 3), (9, 40, 32, 0)]
SPLIT = [(1, 3584, 18944, 16), (1, 64, 8192, 0), (8, 3584, 18944, 16), (40, 264, 544, 8)]


@pytest.mark.parametrize("m,n,k,r", FUSED + SPLIT)
@pytest.mark.parametrize("fmt", [0, 1])
def test_linear_aqn(fp4w, fmt, m, n, k, r):
    what = f"fmt={fmt} m={m} n={n} k={k} r={r}"
    say(f"[linear aqn] {what}")
    x, gamma, noise, codes, scales, st, a, b = _case(m + n + k + r, fmt, m, n, k, r)
    for sigma in (O.aqn_sigma(0, 1000), 0.0):
        got, _ = _run(fp4w, fmt, x, gamma, noise, sigma, 1e-6, codes, scales, st, a, b)
        assert np.isfinite(got).all(), f"{what}: an output was not written"
        _check(fmt, got, x, gamma, noise, sigma, 1e-6, codes, scales, st, a, b, f"{what} sigma={sigma}")


@pytest.mark.parametrize("m", [1, 8])
@pytest.mark.parametrize("fmt", [0, 1])
def test_fused_against_two_launches(fp4w, fmt, m):
    """The fused kernel and the norm-then-linear pair agree to the two roundings
    of x~ they take at different points (2^-8 of sum |x~ w| between them)."""
    n, k, r = 18944, 3584, 16
    x, gamma, noise, codes, scales, st, a, b = _case(3, fmt, m, n, k, r)
    sigma, eps = 1e-2, 1e-6
    got, q = _run(fp4w, fmt, x, gamma, noise, sigma, eps, codes, scales, st, a, b)
    xn = fp4w.aqn_rmsnorm(bf16_dev(x), bf16_dev(gamma), f32_dev(noise), sigma, eps)
    two = fp4w.linear(xn, q, bf16_dev(a), bf16_dev(b))
    torch.cuda.synchronize()
    two = f64_of_bf16(bits_host(two))
    xt = O.aqn_rmsnorm(x, gamma, noise, sigma, eps)
    weff = O.dequantize(fmt, codes, scales, st, "f64") + f64_of_bf16(b) @ f64_of_bf16(a)
    lim = 2 * 2e-3 * np.linalg.norm(xt, axis=1)[:, None] * np.linalg.norm(weff, axis=1)[None, :] \
        + 2.0 ** -7 * (np.abs(xt) @ np.abs(weff).T)
    assert (np.abs(got - two) <= lim).all()
    # repeated calls give the same bits (sums in a fixed order)
    again, _ = _run(fp4w, fmt, x, gamma, noise, sigma, eps, codes, scales, st, a, b)
    assert np.array_equal(got, again)


def test_linear_aqn_zero_rows_and_workspace(fp4w):
    """m = 0 launches nothing; the workspace size covers the norm's buffer where
    the route takes two launches, and a short workspace is refused."""
    n, k = 64, 256
    x, gamma, noise, codes, scales, st, _, _ = _case(1, 0, 5, n, k, 0)
    q = qweight_dev(fp4w, 0, codes, scales, st)
    assert fp4w.linear_aqn_workspace_bytes(5, n, k, 0) >= fp4w.linear_workspace_bytes(5, n, k, 0) + 5 * k * 2
    y = fp4w.linear_aqn(bf16_dev(x[:0]), bf16_dev(gamma), f32_dev(noise), 1e-2, q)
    assert y.shape == (0, n)
    short = torch.zeros(fp4w.linear_workspace_bytes(5, n, k, 0), dtype=torch.uint8, device=DEV)
    with pytest.raises(fp4w.Fp4wError):
        fp4w.linear_aqn(bf16_dev(x), bf16_dev(gamma), f32_dev(noise), 1e-2, q, workspace=short)
