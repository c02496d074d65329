"""GPU parity of the noisy RMSNorm (fp4w_aqn_rmsnorm) against the binary64
oracle: every output within 2^-8 of the oracle's value (one bf16 rounding of an
fp32 computation); in place; sigma = 0 gives the plain RMSNorm."""
import numpy as np
import pytest
import torch

import oracle as O
from mxfp4_bit_weight_amd import workloads as W
from tests.gpu_util import DEV, Guarded, bf16_dev, bits_host, f32_dev, f64_of_bf16, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp4w():
    from mxfp4_bit_weight_amd import fp4w as F
    return F


def _check(got, want, what):
    err = np.abs(got - want)
    bad = ~(err <= 2.0 ** -8 * np.abs(want) + 1e-30)
    assert not bad.any(), f"{what}: {bad.sum()} outputs off, worst {err.max():.3e}"


@pytest.mark.parametrize("m,k", [(1, 3584), (16, 3584), (5, 18944), (3, 8), (7, 1000), (300, 512)])
def test_aqn_rmsnorm(fp4w, m, k):
    say(f"[aqn] m={m} k={k}")
    rng = np.random.default_rng(m + k)
    x = W.to_bf16_bits(rng.standard_normal((m, k)) * 3.0)
    gamma = W.to_bf16_bits(1.0 + 0.1 * rng.standard_normal(k))
    noise = rng.standard_normal(k).astype(np.float32)
    for step in (0, 400, 1000):
        sigma = O.aqn_sigma(step, 1000)
        g = Guarded((m, k), torch.bfloat16, float("nan"))
        y = fp4w.aqn_rmsnorm(bf16_dev(x), bf16_dev(gamma), f32_dev(noise), sigma, 1e-6, out=g.t)
        g.check(f"aqn m={m} k={k}")
        _check(f64_of_bf16(bits_host(y)), O.aqn_rmsnorm(x, gamma, noise, sigma, 1e-6), f"m={m} k={k} step={step}")


def test_aqn_in_place_and_zero_sigma(fp4w):
    rng = np.random.default_rng(9)
    m, k = 8, 2048
    x = W.to_bf16_bits(rng.standard_normal((m, k)))
    gamma = W.to_bf16_bits(rng.standard_normal(k))
    noise = rng.standard_normal(k).astype(np.float32)
    xd = bf16_dev(x)
    fp4w.aqn_rmsnorm(xd, bf16_dev(gamma), f32_dev(noise), 0.0, 1e-5, out=xd)
    torch.cuda.synchronize()
    _check(f64_of_bf16(bits_host(xd)), O.aqn_rmsnorm(x, gamma, np.zeros(k, np.float32), 0.0, 1e-5), "in place, sigma 0")
