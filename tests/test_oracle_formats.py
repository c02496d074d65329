"""Pins of the oracle's scalar codecs against independent formulations.

- E4M3 and E8M0 decoding against PyTorch's float8_e4m3fn / float8_e8m0fnu views.
- E4M3 encoding of exactly representable values against PyTorch's RNE cast.
- E2M1 encoding against a nearest-by-exact-distance search.
- Exact-quotient rounding (the decision the quantizer takes) against Fractions,
  on constructed ties and near-ties.
- bf16 rounding of exact values against a Fraction brute force.
"""
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from tests import exact as X


def test_e2m1_decode_closed_form():
    # OCP E2M1: magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}; bit 3 is the sign.
    for c in range(16):
        mag = X.E2M1_MAGS[c & 7]
        v = O.e2m1_decode(c)
        assert Fraction(abs(v)) == mag
        assert np.signbit(v) == bool(c & 8)


def test_e4m3_decode_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([O.e4m3_decode(c) for c in range(256)])
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))


def test_e8m0_decode_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = np.array([O.e8m0_decode(c) for c in range(256)])
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(ref[:255], got[:255])


def _all_positive_finite_bf16():
    bits = np.arange(0x0000, 0x7F80, dtype=np.uint32)   # +0 .. largest finite
    return (bits << 16).view(np.float32).astype(np.float64)


def test_e4m3_encode_matches_torch_cast_on_exact_values():
    # For a value v exactly representable in binary32, PyTorch's float8_e4m3fn cast
    # rounds to nearest even (it does not saturate, so clamp at 448 first).
    vals = _all_positive_finite_bf16()
    ref = torch.from_numpy(np.minimum(vals, 448.0).astype(np.float32)).to(torch.float8_e4m3fn)
    ref = ref.view(torch.uint8).numpy()
    for d_exp in (0, -7, 5):
        d = 2.0 ** d_exp
        got = np.array([O.e4m3_rne_quot(v, d) for v in vals * d])
        assert np.array_equal(got, ref), d


def test_e2m1_encode_all_bf16_vs_nearest_distance():
    vals = _all_positive_finite_bf16()
    # restrict to the interesting range; everything above 6 saturates
    sel = vals[(vals < 8.0)]
    sel = np.concatenate([sel[::7], sel[-4096:], [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0]])
    for v in sel:
        want = X.nearest_even(Fraction(v), X.E2M1_MAGS)
        assert O.e2m1_rne_quot(v, 1.0) == want, v


def test_e2m1_tie_table():
    # Exact midpoints go to the neighbour with the even code.
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for q, code in ties.items():
        assert O.e2m1_rne_quot(q, 1.0) == code
        # also through a non-power-of-two denominator: q*D exact
        D = 3.75 * 2.0 ** -10
        assert O.e2m1_rne_quot(q * D, D) == code
    assert O.e2m1_rne_quot(100.0, 1.0) == 7           # saturation


def _rand_f32(rng, lo_exp, hi_exp):
    m = rng.randrange(1 << 23, 1 << 24)
    return float(np.float32(m * 2.0 ** (rng.randrange(lo_exp, hi_exp) - 23)))


def test_exact_quotient_decisions_vs_fractions():
    """a/(dec(sb) * s_t) and a/(6 s_t) near and at midpoints, decided exactly."""
    rng = random.Random(1234)
    mids_e2m1 = [(X.E2M1_MAGS[i] + X.E2M1_MAGS[i + 1]) / 2 for i in range(7)]
    mids_e4m3 = [(X.E4M3_MAGS[i] + X.E4M3_MAGS[i + 1]) / 2 for i in range(126)]
    n_checked = 0
    for _ in range(3000):
        st = _rand_f32(rng, -30, 10)
        sb = rng.randrange(1, 0x7F)
        D = float(X.E4M3_MAGS[sb] * Fraction(st))          # <= 28 bits: exact double
        assert Fraction(D) == X.E4M3_MAGS[sb] * Fraction(st)
        mu = rng.choice(mids_e2m1)
        target = mu * Fraction(D)
        # bf16 values at and around the midpoint product
        f = np.float32(float(target))
        bits = int(np.array([f], np.float32).view(np.uint32)[0]) >> 16
        for bb in (bits - 1, bits, bits + 1, bits + 2):
            a = X.bf16_to_fraction(bb)
            want = X.nearest_even(a / Fraction(D), X.E2M1_MAGS)
            assert O.e2m1_rne_quot(float(a), D) == want
            n_checked += 1
        # block scale decision a_b / (6 s_t) around an E4M3 midpoint
        mu4 = rng.choice(mids_e4m3)
        target = mu4 * 6 * Fraction(st)
        f = np.float32(float(target))
        bits = int(np.array([f], np.float32).view(np.uint32)[0]) >> 16
        for bb in (bits - 1, bits, bits + 1):
            a = X.bf16_to_fraction(bb)
            want = X.nearest_even(a / (6 * Fraction(st)), X.E4M3_MAGS)
            assert O.e4m3_rne_quot(float(a), 6.0 * st) == want
            n_checked += 1
    assert n_checked > 10000


def test_exact_ties_with_non_power_of_two_scale():
    # s_t = 3*2^-10, dec(sb) = 1.25 -> S = 3.75*2^-10; every E2M1 midpoint times S is
    # a bf16 value, so these are exact ties and must go to the even code.
    S = 3.75 * 2.0 ** -10
    for mu, code in [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6)]:
        a = mu * S
        assert np.float32(a) == a and (np.array([a], np.float32).view(np.uint32)[0] & 0xFFFF) == 0
        assert O.e2m1_rne_quot(a, S) == code


def _bf16_nearest_even(v: Fraction) -> int:
    """bf16 bit pattern nearest to the exact value v (finite range), ties to even."""
    x32 = np.float32(float(v))
    b = int(np.array([x32], np.float32).view(np.uint32)[0]) >> 16
    cands = []
    for c in (b - 1, b, b + 1):
        if c < 0 or (c & 0x7FFF) >= 0x7F80:
            continue
        cands.append(c)
    best = None
    for c in cands:
        d = abs(X.bf16_to_fraction(c) - v)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def test_round_bf16_vs_fractions():
    rng = random.Random(99)
    for _ in range(20000):
        # products like e2m1 * dec(sb) * s_t: up to 30 significant bits
        m = rng.randrange(1 << 29, 1 << 30)
        e = rng.randrange(-150, 97)
        v = m * 2.0 ** e
        if rng.random() < 0.3:                     # force exact bf16 ties
            v = (rng.randrange(1 << 8, 1 << 9) * 2 + 1) * 2.0 ** (e // 4)
        want = _bf16_nearest_even(Fraction(v))
        assert O.round_bf16(v) == want, v
        assert O.round_bf16(-v) == want | 0x8000
    assert O.round_bf16(0.0) == 0 and O.round_bf16(-0.0) == 0x8000
    assert O.round_bf16(2.0 ** 128) == 0x7F80        # overflow to infinity
    assert O.round_bf16(2.0 ** -134) == 0             # half of the smallest subnormal: tie to 0
    assert O.round_bf16(1.5 * 2.0 ** -134) == 1


def test_mxfp4_scale_code_floor_log2():
    for v in [1.0, 1.5, 2.0, 3.99, 4.0, 6.0, 2.0 ** -126, 2.0 ** -133, 2.0 ** 127 * 1.5]:
        e = X.floor_log2(Fraction(v)) - 2
        assert O.mxfp4_scale_code(v) == max(-127, min(127, e)) + 127
    assert O.mxfp4_scale_code(0.0) == 0
    assert O.mxfp4_scale_code(float("inf")) == 0xFF
    assert O.mxfp4_scale_code(float("nan")) == 0xFF


@pytest.mark.parametrize("a", [0.0, 1e-30, 448.0, 1e9])
def test_tensor_scale_is_binary32_division(a):
    w = X_bf16([a, -a / 2])
    st = O.nvfp4_tensor_scale(w)
    amax = float(np.abs(X_f32(w)).max())
    assert st == np.float32(amax) / np.float32(2688.0)


def X_bf16(vals):
    from mxfp4_bit_weight_amd.workloads import to_bf16_bits
    return to_bf16_bits(np.array(vals, np.float64))


def X_f32(bits):
    from mxfp4_bit_weight_amd.workloads import bf16_bits_to_f32
    return bf16_bits_to_f32(bits)
