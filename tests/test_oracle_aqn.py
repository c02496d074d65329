"""Pins of the noisy RMSNorm (AQN) oracle and its noise schedule: the schedule's
end points and constant ratio (exponential decay), the library's host schedule
against the closed form, a unit-RMS output at sigma = 0, scale invariance, and
the page's equivalence of gain noise with multiplicative noise on the next
projection's weight columns."""
import math

import numpy as np
import pytest

import oracle as O
from mxfp4_bit_weight_amd import workloads as W


def test_schedule_end_points_and_ratio():
    T = 1000
    assert O.aqn_sigma(0, T) == 1e-2 and O.aqn_sigma(T, T) == 5e-4 and O.aqn_sigma(T + 5, T) == 5e-4
    r = [O.aqn_sigma(t + 1, T) / O.aqn_sigma(t, T) for t in range(1, T - 1)]
    assert max(r) - min(r) < 1e-12 and abs(r[0] - (5e-4 / 1e-2) ** (1 / T)) < 1e-12
    assert abs(O.aqn_sigma(T // 2, T) - math.sqrt(1e-2 * 5e-4)) < 1e-15


def test_library_schedule_matches_closed_form():
    from mxfp4_bit_weight_amd import fp4w
    for t in (0, 1, 17, 500, 999, 1000, 2000):
        assert abs(fp4w.aqn_sigma(t, 1000) - O.aqn_sigma(t, 1000)) <= 1e-15
    assert fp4w.aqn_sigma(3, 10, 0.0, 5e-4) == 0.0


def test_zero_noise_is_unit_rms_and_scale_invariant():
    rng = np.random.default_rng(3)
    x = W.to_bf16_bits(rng.standard_normal((4, 256)))
    ones = W.to_bf16_bits(np.ones(256))
    y = O.aqn_rmsnorm(x, ones, np.zeros(256, np.float32), 0.0, 0.0)
    assert np.allclose(np.sqrt((y * y).mean(axis=1)), 1.0, rtol=1e-13)
    x2 = W.to_bf16_bits(2.0 * W.bf16_bits_to_f32(x))                   # exact doubling
    assert np.array_equal(O.aqn_rmsnorm(x2, ones, np.zeros(256, np.float32), 0.0, 0.0), y)


@pytest.mark.parametrize("fmt", [O.NVFP4, O.MXFP4])
def test_gain_noise_is_multiplicative_weight_noise(fmt):
    rng = np.random.default_rng(4)
    w, x, _, _ = W.linear_inputs(5, 48, 128, 3)
    codes, scales, st = O.quantize(fmt, w)
    deq = O.dequantize(fmt, codes, scales, st, "f64")
    gamma = W.to_bf16_bits(1.0 + 0.1 * rng.standard_normal(128))
    noise = rng.standard_normal(128).astype(np.float32)
    sigma = 1e-2
    noisy = O.aqn_rmsnorm(x, gamma, noise, sigma, 1e-6) @ deq.T
    plain = O.aqn_rmsnorm(x, gamma, np.zeros(128, np.float32), 0.0, 1e-6)
    wn = deq * (1.0 + float(np.float32(sigma)) * noise.astype(np.float64))[None, :]
    assert np.allclose(noisy, plain @ wn.T, rtol=1e-12, atol=1e-12 * np.abs(noisy).max())


def test_gain_against_closed_forms():
    """The gain gamma enters once, per channel, as a factor (Telegram post,
    "Metod": the norm ahead of the projections).  Two closed forms pin it:
    a constant row x = c has RMS |c|, so at sigma = 0 and eps = 0 the output is
    sign(c) * gamma exactly; a one-hot row (value v at channel j) has mean square
    v^2 / k, so y_j = sign(v) * sqrt(k) * gamma_j * (1 + sigma * noise_j) and
    every other channel is 0.  A dropped, squared or shifted gamma fails both."""
    k = 64
    gamma_f = np.where(np.arange(k) % 3 == 0, 2.0, 0.5)       # 2 on channels 0, 3, 6, ...; 0.5 elsewhere
    gamma_f[5] = -1.5
    gamma = W.to_bf16_bits(gamma_f)
    zeros = np.zeros(k, np.float32)
    for c in (3.0, -0.75):
        x = W.to_bf16_bits(np.full((1, k), c))
        y = O.aqn_rmsnorm(x, gamma, zeros, 0.0, 0.0)[0]
        assert np.array_equal(y, np.sign(c) * gamma_f)
    rng = np.random.default_rng(11)
    noise = rng.standard_normal(k).astype(np.float32)
    sigma = 1e-2
    for j, v in ((0, 5.0), (5, -2.0), (7, 0.25)):
        row = np.zeros((1, k))
        row[0, j] = v
        y = O.aqn_rmsnorm(W.to_bf16_bits(row), gamma, noise, sigma, 0.0)[0]
        want = np.sign(v) * math.sqrt(k) * gamma_f[j] * (1.0 + float(np.float32(sigma)) * float(noise[j]))
        assert abs(y[j] - want) <= 1e-14 * abs(want)
        others = np.delete(y, j)
        assert np.all(others == 0.0)


@pytest.mark.parametrize("fmt", [O.NVFP4, O.MXFP4])
def test_linear_of_the_norm_against_the_c_linear(fmt):
    """The composition (norm, then projection with its LoRA branch) pinned against
    the C oracle's linear on inputs where the norm's output is exact in bf16:
    rows of +-c (RMS |c|, eps 0) give x~ = +-gamma (1 + sigma noise), and with
    sigma = 1, noise in {0, 1, -1/2} and gamma in {1, 2, -1/2} every factor is a
    power of two.  A norm applied twice, a noise term on the wrong axis, or a
    LoRA branch fed x instead of x~ fails it."""
    rng = np.random.default_rng(21)
    n, k, r = 40, 96, 5
    w, _, a, b = W.linear_inputs(6, n, k, 2, rank=r)
    codes, scales, st = O.quantize(fmt, w)
    gamma_f = rng.choice([1.0, 2.0, -0.5], k)
    noise = rng.choice([0.0, 1.0, -0.5], k).astype(np.float32)
    for c in (3.0, 0.375):
        signs = rng.choice([-1.0, 1.0], (2, k))
        x = W.to_bf16_bits(c * signs)
        xt = signs * gamma_f[None, :] * (1.0 + noise.astype(np.float64))[None, :]
        want = O.linear(fmt, W.to_bf16_bits(xt), codes, scales, st, a, b)
        got = O.linear_aqn(fmt, x, W.to_bf16_bits(gamma_f), noise, 1.0, 0.0, codes, scales, st, a, b)
        assert np.allclose(got, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())
        no_lora = O.linear_aqn(fmt, x, W.to_bf16_bits(gamma_f), noise, 1.0, 0.0, codes, scales, st)
        assert np.allclose(no_lora, O.linear(fmt, W.to_bf16_bits(xt), codes, scales, st), rtol=1e-12,
                           atol=1e-12 * np.abs(want).max())
