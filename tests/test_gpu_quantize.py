"""GPU parity: quantize (NVFP4 dynamic and frozen, MXFP4) must reproduce the
oracle's codes, block scales and tensor scale bit for bit."""
import numpy as np
import pytest
import torch

import oracle as O
from mxfp4_bit_weight_amd import workloads as W
from tests.gpu_util import DEV, guarded_qweight, bf16_dev, f32_dev, qweight_host, say, u8_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp4w():
    from mxfp4_bit_weight_amd import fp4w as F
    return F


def _gpu_quant(fp4w, w_bits, fmt):
    n, k = w_bits.shape
    out, guards = guarded_qweight(fp4w, fmt, n, k)
    q = fp4w.quantize(bf16_dev(w_bits), fmt, out=out)
    for g in guards:
        g.check(f"quantize fmt={fmt} shape={w_bits.shape}")
    return qweight_host(q)


def _compare(fp4w, w_bits, fmt, what):
    say(f"[quantize] {what} fmt={fmt} shape={w_bits.shape}")
    c, s, st = _gpu_quant(fp4w, w_bits, fmt)
    c2, s2, st2 = O.quantize(fmt, w_bits)
    if fmt == O.NVFP4:
        assert np.float32(st).view(np.uint32) == np.float32(st2).view(np.uint32), (st, st2)
    assert np.array_equal(s, s2), f"{what}: {np.sum(s != s2)} block scales differ"
    assert np.array_equal(c, c2), f"{what}: {np.sum(c != c2)} code bytes differ"


@pytest.mark.parametrize("fmt", [0, 1])
def test_single_linear_weight(fp4w, fmt):
    w, _, _, _ = W.linear_inputs(0, 256, 512, 1)
    _compare(fp4w, w, fmt, "single linear 256x512 seed 0")


@pytest.mark.parametrize("name", ["gate_up", "down", "qkv_o"])
@pytest.mark.parametrize("fmt", [0, 1])
def test_full_size_decode_shapes(fp4w, fmt, name):
    shape = W.QWEN7B_SHAPES[name]
    w = W.outlier_weights(1, 0, shape) if fmt == 0 else W.student_t_weights(1, 0, shape)
    _compare(fp4w, w, fmt, f"Qwen-2.5-7B {name} {shape}")


def _near_tie_weights(seed, n, k, st_target):
    """Elements on and one bf16 step either side of E2M1 midpoints times S_b, for
    block scales spread over the E4M3 range, plus the block maxima that fix them."""
    rng = np.random.default_rng(seed)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0])
    vals = rng.standard_normal((n, k)) * st_target * 100
    amax = 2688.0 * st_target
    vals[0, 0] = amax
    codes = torch.arange(0x08, 0x7E, dtype=torch.int32).to(torch.uint8)
    e4 = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for r in range(1, n):
        for b in range(k // 16):
            d = e4[rng.integers(0, e4.size)]
            blk = rng.choice(mids, 16) * d * st_target
            blk[0] = 6.0 * d * st_target                # makes the block scale d (up to rounding)
            vals[r, b * 16:(b + 1) * 16] = blk * rng.choice([-1.0, 1.0], 16)
    bits = W.to_bf16_bits(vals)
    jitter = rng.integers(-1, 2, bits.shape).astype(np.int32)
    jitter[0, 0] = 0
    bits = (bits.astype(np.int32) + jitter).astype(np.uint16)
    return bits


@pytest.mark.parametrize("st_target", [1.0, 2.0 ** -20, 0.0123, 3.0e-7, 2.0 ** 60 / 2688])
def test_near_ties_nvfp4(fp4w, st_target):
    w = _near_tie_weights(5, 64, 512, st_target)
    _compare(fp4w, w, 0, f"near-tie tensor st~{st_target}")


def test_near_ties_mxfp4(fp4w):
    rng = np.random.default_rng(3)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0])
    vals = rng.choice(mids, (64, 512)) * np.exp2(rng.integers(-30, 30, (64, 512 // 32)).repeat(32, axis=1))
    bits = W.to_bf16_bits(vals * rng.choice([-1.0, 1.0], vals.shape))
    bits = (bits.astype(np.int32) + rng.integers(-1, 2, bits.shape)).astype(np.uint16)
    _compare(fp4w, bits, 1, "MXFP4 near-tie tensor")


@pytest.mark.parametrize("fmt", [0, 1])
def test_special_values(fp4w, fmt):
    rng = np.random.default_rng(11)
    vals = rng.standard_normal((8, 256)) * 0.02
    vals[1] = 0.0                                  # zero row
    vals[2, :32] = -0.0
    vals[3, :64] = 2.0 ** -130 * rng.integers(1, 8, 64)   # bf16 subnormals
    vals[4, :32] = 3.0e38 * rng.choice([-1, 1], 32)       # near the bf16 maximum
    vals[5, 16:32] = 1.0e-12                        # a block far below the tensor maximum
    vals[6] = rng.standard_normal(256) * 1e-30
    bits = W.to_bf16_bits(vals)
    bits[2, :32] = 0x8000
    _compare(fp4w, bits, fmt, "special values")


@pytest.mark.parametrize("fmt", [0, 1])
def test_tiny_and_zero_tensors(fp4w, fmt):
    rng = np.random.default_rng(12)
    tiny = W.to_bf16_bits(rng.standard_normal((4, 64)) * 1e-22)     # s_t below 2^-64
    _compare(fp4w, tiny, fmt, "tiny tensor")
    sub = W.to_bf16_bits(rng.standard_normal((4, 64)) * 2.0 ** -128)  # s_t subnormal
    _compare(fp4w, sub, fmt, "subnormal tensor")
    z = np.zeros((4, 64), np.uint16)
    z[1, 5] = 0x8000
    _compare(fp4w, z, fmt, "zero tensor")


def test_nonfinite_is_signalled(fp4w):
    w = W.to_bf16_bits(np.ones((2, 64)))
    w[1, 7] = 0x7F80                                 # +inf
    c, s, st = _gpu_quant(fp4w, w, 0)
    assert not np.isfinite(st)
    c, s, st = _gpu_quant(fp4w, w, 1)
    assert s[1, 0] == 0xFF and s[0, 0] != 0xFF
    w[1, 9] = 0x7FC1                                 # NaN
    c, s, st = _gpu_quant(fp4w, w, 0)
    assert np.isnan(st)


@pytest.mark.parametrize("fmt", [0, 1])
def test_frozen_scales(fp4w, fmt):
    say(f"[quantize] frozen fmt={fmt}")
    w = W.outlier_weights(7, 0, (300, 1024), p=0.01)
    q = fp4w.quantize(bf16_dev(w), fmt)
    q2 = fp4w.quantize(bf16_dev(w), fmt, frozen=q)        # same scales -> same codes
    torch.cuda.synchronize()
    assert torch.equal(q.codes, q2.codes)
    # arbitrary valid scales and tensor scale
    rng = np.random.default_rng(8)
    top = 0x7E if fmt == 0 else 0xFE
    scales = rng.integers(0, top + 1, q.scales.shape).astype(np.uint8)
    if fmt == 1:
        scales = rng.integers(100, 140, q.scales.shape).astype(np.uint8)
    st = np.float32(3.7e-5)
    frozen = fp4w.QWeight(fmt, None, u8_dev(scales), f32_dev([st]) if fmt == 0 else None, 300, 1024)
    out = fp4w.empty_qweight(fmt, 300, 1024, DEV)
    q3 = fp4w.quantize(bf16_dev(w), fmt, out=out, frozen=frozen)
    torch.cuda.synchronize()
    want = O.quantize_frozen(fmt, w, scales, st)
    got = q3.codes.cpu().numpy()
    assert np.array_equal(got, want), f"{np.sum(got != want)} code bytes differ"
    assert np.array_equal(q3.scales.cpu().numpy(), scales)          # scales untouched


def test_tensor_scale_every_bf16_amax(fp4w):
    """s_t = fl32(A / 2688) for every finite non-negative bf16 amax (32640 values),
    plus block scales and codes of each one-row tensor."""
    say("[quantize] exhaustive tensor scale")
    amax_bits = np.arange(0x0001, 0x7F80, dtype=np.uint32)
    n = amax_bits.size
    rng = np.random.default_rng(2)
    amax = (amax_bits << 16).view(np.float32).astype(np.float64)
    rows = rng.uniform(-1, 1, (n, 32)) * amax[:, None]
    w = W.to_bf16_bits(rows)
    w[:, 0] = amax_bits.astype(np.uint16)                     # the row maximum, exactly
    w = np.where((w & 0x7FFF) > amax_bits[:, None], amax_bits[:, None].astype(np.uint16), w).astype(np.uint16)
    wd = bf16_dev(w)
    codes = torch.empty((n, 16), dtype=torch.uint8, device=DEV)
    scales = torch.empty((n, 2), dtype=torch.uint8, device=DEV)
    ts = torch.empty(n, dtype=torch.float32, device=DEV)
    stream = torch.cuda.current_stream().cuda_stream
    import ctypes
    for i in range(n):
        rc = fp4w._quantize(0, ctypes.c_void_p(wd.data_ptr() + 64 * i), 1, 32,
                            ctypes.c_void_p(codes.data_ptr() + 16 * i), ctypes.c_void_p(scales.data_ptr() + 2 * i),
                            ctypes.c_void_p(ts.data_ptr() + 4 * i), 0, ctypes.c_void_p(stream))
        assert rc == 0
    torch.cuda.synchronize()
    got = ts.cpu().numpy()
    want = (np.float32(1.0) * amax.astype(np.float32)) / np.float32(2688.0)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    c_got, s_got = codes.cpu().numpy(), scales.cpu().numpy()
    bad = 0
    for i in range(0, n, 7):
        c2, s2 = O.nvfp4_quantize_with_tensor_scale(w[i:i + 1], want[i])
        bad += int(not (np.array_equal(c2[0], c_got[i]) and np.array_equal(s2[0], s_got[i])))
    assert bad == 0


def test_tensor_scale_across_calls_and_streams(fp4w):
    """The amax is reduced in a slot the library holds per stream and returns to
    zero after every call: a run of tensors whose maxima fall (a slot that kept a
    maximum would give every later tensor the first one's scale), tensors big
    enough for many reducing workgroups, and calls interleaved on two streams
    without synchronisation, each against the oracle's tensor scale, bit for bit."""
    say("[quantize] tensor scale across calls and streams")
    rng = np.random.default_rng(12)
    shapes = [(64, 256), (512, 1024), (3584, 3584), (40, 96)]
    ws, wants = [], []
    for i in range(24):
        n, k = shapes[i % len(shapes)]
        w = W.to_bf16_bits(rng.standard_normal((n, k)) * 2.0 ** (-i / 3.0))
        ws.append(w)
        wants.append(O.nvfp4_tensor_scale(w))
    dev_w = [bf16_dev(w) for w in ws]
    torch.cuda.synchronize()
    outs = [fp4w.quantize(dw, 0) for dw in dev_w]           # falling maxima on one stream
    torch.cuda.synchronize()
    for i, q in enumerate(outs):
        assert np.float32(q.tensor_scale.item()).view(np.uint32) == np.float32(wants[i]).view(np.uint32), i
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = [None] * len(dev_w)
    for i, dw in enumerate(dev_w):
        with torch.cuda.stream(s1 if i % 2 == 0 else s2):
            outs[i] = fp4w.quantize(dw, 0)
    torch.cuda.synchronize()
    for i, q in enumerate(outs):
        assert np.float32(q.tensor_scale.item()).view(np.uint32) == np.float32(wants[i]).view(np.uint32), i
    c, s, st = qweight_host(outs[2])
    c2, s2_, _ = O.quantize(0, ws[2])
    assert np.array_equal(c, c2) and np.array_equal(s, s2_)
