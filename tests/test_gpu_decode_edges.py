"""Edge cases of the decode path (m <= 8), which feeds x to the block-scaled
matrix core as two E4M3 terms per element under an E8M0 scale per 32 elements:

- activations spanning many binades inside one block, bf16 subnormals, zero
  blocks and rows far below 1 stay within |err| <= 2e-3 ||x_m|| ||w_n^eff||;
- a non-finite activation turns every output of its row NaN and leaves the other
  rows untouched;
- scale bytes that start at an odd 2-byte offset (staged byte by byte).
"""
import numpy as np
import pytest
import torch

import oracle as O
from mxfp4_bit_weight_amd import workloads as W
from tests.gpu_util import (DEV, bf16_dev, bits_host, check_bound, f64_of_bf16, qweight_dev, say, u8_dev,
                            weff_norms)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp4w():
    from mxfp4_bit_weight_amd import fp4w as F
    return F


def _bf16_bits(v: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bits, round to nearest even (finite inputs)."""
    f = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (f + 0x7FFF + ((f >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def _wide_range_x(seed: int, m: int, k: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, k))
    # per element a random binade in [-40, 0] relative to the row, so most 32-blocks
    # hold elements far below their block maximum
    x *= np.exp2(-rng.integers(0, 41, (m, k)).astype(np.float64))
    x[:, 64:96] = 0.0                                       # an all-zero block
    if m > 1:
        x[1] *= 1e-30                                       # a row far below 1
    if m > 2:
        x[2, :32] = rng.standard_normal(32) * 1e-39         # bf16 subnormals
    return _bf16_bits(x)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("m", [1, 3, 8])
def test_wide_dynamic_range_activations(fp4w, fmt, m):
    n, k = 300, 2080
    say(f"[decode-edges] wide-range x fmt={fmt} m={m}")
    w, _, a, b = W.linear_inputs(61 + m, n, k, m, rank=16, wkind="outlier")
    x = _wide_range_x(62 + m, m, k)
    codes, scales, st = O.quantize(fmt, w)
    q = qweight_dev(fp4w, fmt, codes, scales, st)
    y = fp4w.linear(bf16_dev(x), q, bf16_dev(a), bf16_dev(b))
    torch.cuda.synchronize()
    yg = f64_of_bf16(bits_host(y))
    y64 = O.linear(fmt, x, codes, scales, st, a, b)
    xn = np.sqrt((f64_of_bf16(x) ** 2).sum(axis=1))[:, None]
    wn = weff_norms(fmt, codes, scales, st, a, b)[None, :]
    check_bound(yg, y64, xn, wn, f"wide-range x m={m}")


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("bad", [np.inf, -np.inf, np.nan])
def test_non_finite_activation_poisons_its_row_only(fp4w, fmt, bad):
    m, n, k = 4, 200, 544
    say(f"[decode-edges] non-finite x fmt={fmt} value={bad}")
    w, x, a, b = W.linear_inputs(71, n, k, m, rank=16)
    x = x.copy()
    x[2, 100] = 0x7F80 if bad == np.inf else (0xFF80 if bad == -np.inf else 0x7FC0)
    codes, scales, st = O.quantize(fmt, w)
    q = qweight_dev(fp4w, fmt, codes, scales, st)
    y = fp4w.linear(bf16_dev(x), q, bf16_dev(a), bf16_dev(b)).float().cpu().numpy()
    assert np.isnan(y[2]).all()
    keep = [0, 1, 3]
    y64 = O.linear(fmt, x[keep], codes, scales, st, a, b)
    xn = np.sqrt((f64_of_bf16(x[keep]) ** 2).sum(axis=1))[:, None]
    wn = weff_norms(fmt, codes, scales, st, a, b)[None, :]
    check_bound(y[keep].astype(np.float64), y64, xn, wn, "rows without the non-finite element")


def test_nvfp4_scales_at_odd_two_byte_offset(fp4w):
    m, n, k = 2, 130, 1056
    say("[decode-edges] NVFP4 scales at a 2-byte offset")
    w, x, a, b = W.linear_inputs(81, n, k, m, rank=8)
    codes, scales, st = O.quantize(0, w)
    q = qweight_dev(fp4w, 0, codes, scales, st)
    buf = torch.zeros(scales.size + 64, dtype=torch.uint8, device=DEV)
    view = buf[2:2 + scales.size].view(n, k // 16)
    view.copy_(u8_dev(scales))
    q2 = fp4w.QWeight(0, q.codes, view, q.tensor_scale, n, k)
    y_off = fp4w.linear(bf16_dev(x), q2, bf16_dev(a), bf16_dev(b))
    y_ref = fp4w.linear(bf16_dev(x), q, bf16_dev(a), bf16_dev(b))
    torch.cuda.synchronize()
    assert torch.equal(y_off.view(torch.int16), y_ref.view(torch.int16))
