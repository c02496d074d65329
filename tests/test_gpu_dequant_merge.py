"""GPU parity: dequantize (bf16 and fp32 outputs) and the scale-only merge must be
bit-exact with the oracle; the merge's code plane must be byte-identical."""
import numpy as np
import pytest
import torch

import oracle as O
from mxfp4_bit_weight_amd import workloads as W
from tests.gpu_util import DEV, Guarded, bits_host, bf16_dev, f32_dev, qweight_dev, say, u8_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp4w():
    from mxfp4_bit_weight_amd import fp4w as F
    return F


def _dequant_both(fp4w, fmt, codes, scales, st, what):
    say(f"[dequantize] {what} fmt={fmt} shape={codes.shape}")
    q = qweight_dev(fp4w, fmt, codes, scales, st)
    n, k = codes.shape[0], codes.shape[1] * 2
    gb_, gf_ = Guarded((n, k), torch.bfloat16), Guarded((n, k), torch.float32)
    yb = fp4w.dequantize(q, torch.bfloat16, out=gb_.t)
    yf = fp4w.dequantize(q, torch.float32, out=gf_.t)
    gb_.check(f"dequantize bf16 {what}")
    gf_.check(f"dequantize fp32 {what}")
    gb, gf = bits_host(yb), yf.cpu().numpy()
    wb = O.dequantize(fmt, codes, scales, st, "bf16")
    wf = O.dequantize(fmt, codes, scales, st, "f32")
    assert np.array_equal(gb, wb), f"{what}: {np.sum(gb != wb)} bf16 values differ"
    assert np.array_equal(gf.view(np.uint32), wf.view(np.uint32)), \
        f"{what}: {np.sum(gf.view(np.uint32) != wf.view(np.uint32))} fp32 values differ"


@pytest.mark.parametrize("fmt", [0, 1])
def test_dequant_quantized_full_size(fp4w, fmt):
    w = W.outlier_weights(2, 0, W.QWEN7B_SHAPES["gate_up"])
    codes, scales, st = O.quantize(fmt, w)
    _dequant_both(fp4w, fmt, codes, scales, st, "gate_up full size")


# tensor scales chosen to land products on and next to bf16 ties, plus tiny ones
ST_VALUES = [1.0, 1.00390625, 1.0 + 2.0 ** -8 + 2.0 ** -23, 0.3333333, 7.1e-5, 2.0 ** -100, 1.5e-42, 3.0e30]


@pytest.mark.parametrize("st", ST_VALUES)
def test_dequant_every_code_and_scale_nvfp4(fp4w, st):
    # row s (scale byte s) holds all 16 codes in both nibble positions
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 2, axis=1)      # k = 32: 2 blocks
    base = np.arange(16, dtype=np.uint8)
    codes = np.tile((base | (base[::-1] << 4)), (256, 1))                       # 16 bytes = 32 codes
    _dequant_both(fp4w, 0, codes, scales, np.float32(st), f"all codes x scales st={st}")


def test_dequant_every_code_and_scale_mxfp4(fp4w):
    scales = np.arange(256, dtype=np.uint8)[:, None]
    base = np.arange(16, dtype=np.uint8)
    codes = np.tile((base | (base[::-1] << 4)), (256, 1))
    _dequant_both(fp4w, 1, codes, scales, np.float32(1.0), "MXFP4 all codes x scales")


@pytest.mark.parametrize("fmt", [0, 1])
def test_dequant_random_codes_many_scales(fp4w, fmt):
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 256, (512, 256), dtype=np.uint8)
    top = 0x7E if fmt == 0 else 0xFE
    scales = rng.integers(0, top + 1, (512, 512 // O.BLOCK[fmt]), dtype=np.uint8)
    _dequant_both(fp4w, fmt, codes, scales, np.float32(0.0123456), "random codes and scales")


def _merge_case(fp4w, fmt, scales, deltas, what, codes=None):
    say(f"[merge] {what} fmt={fmt} blocks={scales.size}")
    if codes is None:
        codes = np.random.default_rng(0).integers(0, 256, (scales.shape[0], 16), dtype=np.uint8)
    q = qweight_dev(fp4w, fmt, codes, scales, np.float32(0.5))
    d = f32_dev(deltas.reshape(scales.shape))
    new = fp4w.merge_scales(q, d)                      # out of place: codes copied
    gso = Guarded(scales.shape, torch.uint8)
    fp4w.merge_scales(q, d, scales_out=gso.t)
    gso.check(f"merge {what}")
    torch.cuda.synchronize()
    want, _ = O.merge_scales(fmt, scales, deltas)
    got = new.scales.cpu().numpy()
    assert np.array_equal(got.reshape(-1), want.reshape(-1)), f"{what}: {np.sum(got.reshape(-1) != want.reshape(-1))} differ"
    assert new.codes.cpu().numpy().tobytes() == codes.tobytes()
    assert new.codes.data_ptr() != q.codes.data_ptr()
    if fmt == 0:
        assert new.tensor_scale.data_ptr() == q.tensor_scale.data_ptr()
    q_in = qweight_dev(fp4w, fmt, codes, scales, np.float32(0.5))
    fp4w.merge_scales(q_in, d, in_place=True)
    torch.cuda.synchronize()
    assert np.array_equal(q_in.scales.cpu().numpy().reshape(-1), want.reshape(-1))
    assert q_in.codes.cpu().numpy().tobytes() == codes.tobytes()


@pytest.mark.parametrize("fmt", [0, 1])
def test_merge_full_size_scales(fp4w, fmt):
    """Scale-only update of the (18944, 3584) weight: deltas ~ N(0, 0.05 s)."""
    w = W.outlier_weights(3, 0, W.QWEN7B_SHAPES["gate_up"])
    codes, scales, st = O.quantize(fmt, w)
    z = W.merge_noise(3, scales.size)
    s_t = torch.from_numpy(scales.reshape(-1))
    dec = (s_t.view(torch.float8_e4m3fn) if fmt == 0 else s_t.view(torch.float8_e8m0fnu)).to(torch.float32).numpy()
    deltas = (np.float32(0.05) * dec * z).astype(np.float32)
    _merge_case(fp4w, fmt, scales, deltas, "gate_up scales", codes=codes)


def test_merge_constructed_ties_nvfp4(fp4w):
    e4 = torch.arange(0x7F, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    rng = np.random.default_rng(6)
    n = 20000
    c = rng.integers(0, 0x7F, n)
    j = rng.integers(0, 0x7E, n)
    target = 0.5 * (e4[j] + e4[j + 1])
    d = (target - e4[c]).astype(np.float32)            # exact for most pairs
    d[::5] = np.nextafter(d[::5], np.float32(np.inf))
    d[1::5] = np.nextafter(d[1::5], -np.float32(np.inf))
    d[2::97] = np.nan
    d[3::89] = -1e30
    d[4::83] = np.inf
    scales = c.astype(np.uint8).reshape(-1, 2)
    _merge_case(fp4w, 0, scales, d.reshape(-1), "NVFP4 constructed ties")


def test_merge_every_e4m3_midpoint(fp4w):
    """Every midpoint of the E4M3 grid (subnormal and normal), reached from the
    codes on both sides and from 0 with deltas nudged by 0, +-1 and +-2 units in
    the last place: the binary32 sum lands on the midpoint with a nonzero
    remainder (the exact path decides), on it exactly (ties to even), or beside it."""
    e4 = torch.arange(0x7F, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    c_list, d_list = [], []
    for j in range(0x7E):
        target = 0.5 * (e4[j] + e4[j + 1])
        for c in (j, j + 1, 0):
            d0 = np.float32(target - e4[c])
            for nudge in (0, 1, -1, 2, -2):
                d = d0
                for _ in range(abs(nudge)):
                    d = np.nextafter(d, np.float32(np.inf) if nudge > 0 else -np.float32(np.inf))
                c_list.append(c)
                d_list.append(d)
    pad = (-len(c_list)) % 2
    c_list += [0] * pad
    d_list += [np.float32(0)] * pad
    scales = np.array(c_list, dtype=np.uint8).reshape(-1, 2)
    _merge_case(fp4w, 0, scales, np.array(d_list, dtype=np.float32), "NVFP4 every midpoint")


def test_merge_constructed_ties_mxfp4(fp4w):
    rng = np.random.default_rng(7)
    n = 20000
    c = rng.integers(0, 255, n)
    j = rng.integers(0, 254, n)
    target = 1.5 * np.exp2(j - 127.0)
    d = (target - np.exp2(c - 127.0)).astype(np.float32)
    d[::4] = np.nextafter(d[::4], np.float32(np.inf))
    d[1::7] = (rng.standard_normal(d[1::7].size) * 1e-3).astype(np.float32)
    d[2::101] = np.nan
    scales = c.astype(np.uint8).reshape(-1, 1)
    scales[5] = 0xFF
    _merge_case(fp4w, 1, scales, d, "MXFP4 constructed ties")


@pytest.mark.parametrize("offsets", [(0, 0, 0), (1, 4, 3), (4, 16, 0), (0, 8, 4)])
def test_merge_unaligned_and_tails(fp4w, offsets):
    """Scale, delta and output pointers at byte offsets that take the merge off its
    16-byte path (and on it), block counts with ragged tails after the whole
    1024-block chunks; canary bytes after the output stay untouched."""
    so, do, oo = offsets
    for nb in (4096 + 1023, 9000, 70001):
        rng = np.random.default_rng(nb + so)
        scales = rng.integers(0, 0x7F, nb, dtype=np.uint8)
        dec = torch.from_numpy(scales).view(torch.float8_e4m3fn).to(torch.float32).numpy()
        deltas = (np.float32(0.05) * dec * rng.standard_normal(nb).astype(np.float32)).astype(np.float32)
        want, _ = O.merge_scales(0, scales, deltas)
        s_buf = torch.zeros(nb + 64, dtype=torch.uint8, device=DEV)
        s_buf[so:so + nb] = u8_dev(scales)
        d_buf = torch.zeros(nb + 64, dtype=torch.float32, device=DEV)
        d_bytes = d_buf.view(torch.uint8)
        d_bytes[do:do + 4 * nb] = u8_dev(deltas.view(np.uint8))
        o_buf = torch.full((nb + 64,), 0xA5, dtype=torch.uint8, device=DEV)
        st = fp4w._merge(0, s_buf.data_ptr() + so, d_buf.data_ptr() + do, nb, o_buf.data_ptr() + oo, None, None, 0,
                         fp4w._stream(DEV))
        assert st == 0
        torch.cuda.synchronize()
        out = o_buf.cpu().numpy()
        assert np.array_equal(out[oo:oo + nb], want.reshape(-1)), f"offsets {offsets} nb={nb}"
        assert (out[:oo] == 0xA5).all() and (out[oo + nb:] == 0xA5).all(), "bytes outside the output were written"
