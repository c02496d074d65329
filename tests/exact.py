"""Exact-rational brute-force formulations used to pin the oracle.

These are written independently of the oracle's C code: values are Python
``Fraction``s, rounding picks the nearest grid value by exact distance (ties to
the even code), and nothing here compares against midpoints or uses binary64
products.  Bit layouts follow the OCP definitions (E2M1, E4M3 "FN", E8M0).
"""
from fractions import Fraction

import numpy as np
import torch

# E2M1 magnitudes by code 0..7 (OCP Microscaling v1.0 element format table).
E2M1_MAGS = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2),
             Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def e4m3_mags():
    """Non-negative E4M3FN values by code 0x00..0x7E, from PyTorch's float8_e4m3fn."""
    codes = torch.arange(0x7F, dtype=torch.int32).to(torch.uint8)
    vals = codes.view(torch.float8_e4m3fn).to(torch.float64).tolist()
    return [Fraction(v) for v in vals]


E4M3_MAGS = e4m3_mags()


def bf16_to_fraction(bits: int) -> Fraction:
    f = np.array([int(bits) << 16], dtype=np.uint32).view(np.float32)[0]
    return Fraction(float(f))


def f32_to_fraction(x) -> Fraction:
    return Fraction(float(np.float32(x)))


def nearest_even(q: Fraction, mags) -> int:
    """Index of the grid value nearest to q; ties to the even index; above the
    top saturates (the top is the nearest by distance anyway)."""
    best, best_d = None, None
    for i, g in enumerate(mags):
        d = abs(q - g)
        if best is None or d < best_d or (d == best_d and i % 2 == 0):
            best, best_d = i, d
    return best


def floor_log2(q: Fraction) -> int:
    e = 0
    while q >= 2:
        q /= 2
        e += 1
    while q < 1:
        q *= 2
        e -= 1
    return e


def nvfp4_quantize_exact(w_bits: np.ndarray):
    """Independent NVFP4 quantize of a small (n, k) bf16 tensor."""
    n, k = w_bits.shape
    vals = [[bf16_to_fraction(b) for b in row] for row in w_bits.tolist()]
    A = max(abs(v) for row in vals for v in row)
    st = np.float32(float(A)) / np.float32(2688.0)      # IEEE binary32 division
    stq = f32_to_fraction(st)
    codes = np.zeros((n, k), np.uint8)
    scales = np.zeros((n, k // 16), np.uint8)
    for r in range(n):
        for b in range(k // 16):
            blk = vals[r][b * 16:(b + 1) * 16]
            ab = max(abs(v) for v in blk)
            sb = 0 if stq == 0 else nearest_even(ab / (6 * stq), E4M3_MAGS)
            scales[r, b] = sb
            S = E4M3_MAGS[sb] * stq
            for j, v in enumerate(blk):
                sign = 8 if (int(w_bits[r, b * 16 + j]) >> 15) & 1 else 0
                mag = 0 if S == 0 else nearest_even(abs(v) / S, E2M1_MAGS)
                codes[r, b * 16 + j] = sign | mag
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, scales, st


def mxfp4_quantize_exact(w_bits: np.ndarray):
    n, k = w_bits.shape
    codes = np.zeros((n, k), np.uint8)
    scales = np.zeros((n, k // 32), np.uint8)
    for r in range(n):
        for b in range(k // 32):
            bits = w_bits[r, b * 32:(b + 1) * 32].tolist()
            blk = [bf16_to_fraction(x) for x in bits]
            ab = max(abs(v) for v in blk)
            e = -127 if ab == 0 else max(-127, min(127, floor_log2(ab) - 2))
            scales[r, b] = e + 127
            D = Fraction(2) ** e
            for j, (v, bb) in enumerate(zip(blk, bits)):
                sign = 8 if (bb >> 15) & 1 else 0
                codes[r, b * 32 + j] = sign | nearest_even(abs(v) / D, E2M1_MAGS)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, scales


def unpack(codes: np.ndarray) -> np.ndarray:
    """(n, k/2) bytes -> (n, k) nibbles, element k in the low nibble when k is even."""
    out = np.empty((codes.shape[0], codes.shape[1] * 2), np.uint8)
    out[:, 0::2] = codes & 0xF
    out[:, 1::2] = codes >> 4
    return out
