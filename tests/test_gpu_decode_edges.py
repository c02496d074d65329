"""Edge cases of the decode paths (m <= 16).  One row of x goes to the
block-scaled matrix core as two E4M3 terms per element under an E8M0 scale per
32 elements; 2 to 16 rows go to the fp16 (NVFP4) or bf16 (MXFP4) matrix core
with x scaled by a power of two per row and wave (NVFP4) and the weights
decoded exactly in registers:

- activations spanning many binades inside one block, bf16 subnormals, zero
  blocks and rows far below 1 stay within |err| <= 2e-3 ||x_m|| ||w_n^eff||;
- a non-finite activation turns every output of its row NaN and leaves the other
  rows untouched;
- a NaN block scale turns every output of its weight row (output column) NaN;
- scale bytes that start at an odd 2-byte or an odd byte offset, and LoRA B rows
  that are not 16-byte aligned.
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
@pytest.mark.parametrize("m", [1, 3, 8, 16])
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


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("m", [1, 5])
def test_nan_block_scale_poisons_its_column_only(fp4w, fmt, m):
    n, k = 70, 640
    say(f"[decode-edges] NaN block scale fmt={fmt} m={m}")
    w, x, a, b = W.linear_inputs(91 + m, n, k, m, rank=16)
    codes, scales, st = O.quantize(fmt, w)
    scales = scales.copy()
    scales[33, 3] = 0x7F if fmt == 0 else 0xFF          # the format's NaN scale code
    q = qweight_dev(fp4w, fmt, codes, scales, st)
    y = fp4w.linear(bf16_dev(x), q, bf16_dev(a), bf16_dev(b)).float().cpu().numpy()
    assert np.isnan(y[:, 33]).all()
    keep = np.array([c for c in range(n) if c != 33])
    y64 = O.linear(fmt, x, codes, scales, st, a, b)[:, keep]
    xn = np.sqrt((f64_of_bf16(x) ** 2).sum(axis=1))[:, None]
    wn = weff_norms(fmt, codes[keep], scales[keep], st, a, b[keep])[None, :]
    check_bound(y[:, keep].astype(np.float64), y64, xn, wn, "columns without the NaN scale")


@pytest.mark.parametrize("fmt", [0, 1])
def test_scales_at_odd_byte_offset(fp4w, fmt):
    """MXFP4 scales may start at any byte; NVFP4 scales must be 2-byte aligned
    and an odd address is refused before anything is launched."""
    m, n, k = 3, 130, 1056
    say(f"[decode-edges] scales at a 1-byte offset fmt={fmt}")
    w, x, a, b = W.linear_inputs(83, n, k, m, rank=8)
    codes, scales, st = O.quantize(fmt, w)
    q = qweight_dev(fp4w, fmt, codes, scales, st)
    buf = torch.zeros(scales.size + 64, dtype=torch.uint8, device=DEV)
    view = buf[1:1 + scales.size].view(scales.shape)
    view.copy_(u8_dev(scales))
    q2 = fp4w.QWeight(fmt, q.codes, view, q.tensor_scale, n, k)
    if fmt == 0:
        with pytest.raises(fp4w.Fp4wError) as ei:
            fp4w.linear(bf16_dev(x), q2, bf16_dev(a), bf16_dev(b))
        assert ei.value.status == -3
        return
    y_off = fp4w.linear(bf16_dev(x), q2, bf16_dev(a), bf16_dev(b))
    y_ref = fp4w.linear(bf16_dev(x), q, bf16_dev(a), bf16_dev(b))
    torch.cuda.synchronize()
    assert torch.equal(y_off.view(torch.int16), y_ref.view(torch.int16))


@pytest.mark.parametrize("m", [1, 6])
def test_lora_b_not_16_byte_aligned(fp4w, m):
    n, k, r = 150, 512, 16
    say(f"[decode-edges] LoRA B at a 2-byte offset m={m}")
    w, x, a, b = W.linear_inputs(87, n, k, m, rank=r)
    codes, scales, st = O.quantize(0, w)
    q = qweight_dev(fp4w, 0, codes, scales, st)
    buf = torch.zeros(b.size + 8, dtype=torch.bfloat16, device=DEV)
    bv = buf[1:1 + b.size].view(n, r)
    bv.copy_(bf16_dev(b))
    y_off = fp4w.linear(bf16_dev(x), q, bf16_dev(a), bv)
    y_ref = fp4w.linear(bf16_dev(x), q, bf16_dev(a), bf16_dev(b))
    torch.cuda.synchronize()
    assert torch.equal(y_off.view(torch.int16), y_ref.view(torch.int16))


@pytest.mark.parametrize("fmt", [0, 1])
def test_codes_beyond_2gib_on_the_fallback_decode(fp4w, fmt):
    """9 rows of x against W (16400, 262144): 2.15e9 bytes of codes, past the
    32-bit buffer offsets of the x-in-registers kernel, so the call runs the
    fallback decode (t = x A^T by its own launch, then the bf16-MFMA decode
    tile).  Random codes under random valid scales (codes and scales drawn
    directly: quantizing a 4.3e9-weight bf16 tensor on the host would take
    minutes); 512 sampled outputs against the oracle, every output written."""
    m, n, k, r = 9, 16400, 262144, 16
    assert n * (k // 2) >= 1 << 31
    say(f"[decode-edges] codes beyond 2 GiB fmt={fmt} m={m} n={n} k={k}")
    g = np.random.default_rng(71 + fmt)
    codes = g.integers(0, 256, (n, k // 2), dtype=np.uint8)
    if fmt == 0:
        scales = g.integers(0x20, 0x48, (n, k // 16), dtype=np.uint8)      # E4M3 2^-3 .. 2^2
        st = np.float32(1.0 / 64)
    else:
        scales = g.integers(120, 130, (n, k // 32), dtype=np.uint8)
        st = np.float32(1.0)
    _, x, a, b = W.linear_inputs(72, 16, k, m, rank=r)
    b = W.normal_bf16(72, W.TID_B, (n, r), 0.01)
    q = qweight_dev(fp4w, fmt, codes, scales, st)
    y = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=DEV)
    fp4w.linear(bf16_dev(x), q, bf16_dev(a), bf16_dev(b), out=y)
    torch.cuda.synchronize()
    del q
    assert bool(torch.isfinite(y).all().item()), "an output was not written"
    rows = g.integers(0, m, 512)
    cols = g.integers(0, n, 512)
    ys = f64_of_bf16(bits_host(y[torch.from_numpy(rows).to(DEV), torch.from_numpy(cols).to(DEV)]))
    y64 = O.linear_sampled(fmt, x, codes, scales, st, rows, cols, a, b)
    xn = np.sqrt((f64_of_bf16(x[rows]) ** 2).sum(axis=1))
    wn = weff_norms(fmt, codes, scales, st, a, b, rows=cols)
    check_bound(ys, y64, xn, wn, "codes beyond 2 GiB")
