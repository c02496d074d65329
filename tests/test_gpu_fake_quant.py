"""GPU parity of the fused fake-quant forward (fp4w_fake_quant): bit for bit the
oracle's dequantize(quantize(W)) rounded to bf16, with the block scales (and
NVFP4 tensor scale) the oracle's quantize gives; frozen scales; the
straight-through backward passes the gradient unchanged."""
import numpy as np
import pytest
import torch

import oracle as O
from mxfp4_bit_weight_amd import workloads as W
from tests.gpu_util import DEV, Guarded, bf16_dev, bits_host, f32_dev, say, u8_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp4w():
    from mxfp4_bit_weight_amd import fp4w as F
    return F


def _compare(fp4w, w_bits, fmt, what):
    say(f"[fake-quant] {what} fmt={fmt} shape={w_bits.shape}")
    g = Guarded(w_bits.shape, torch.bfloat16, float("nan"))
    y, scales, ts = fp4w.fake_quant(bf16_dev(w_bits), fmt, out=g.t)
    g.check(f"fake-quant {what}")
    codes, s2, st2 = O.quantize(fmt, w_bits)
    want = O.dequantize(fmt, codes, s2, st2, "bf16")
    got = bits_host(y)
    assert np.array_equal(scales.cpu().numpy(), s2), f"{what}: block scales differ"
    if fmt == O.NVFP4:
        st = np.float32(ts.item())
        assert st.view(np.uint32) == np.float32(st2).view(np.uint32), (st, st2)
    assert np.array_equal(got, want), f"{what}: {np.sum(got != want)} values differ"


@pytest.mark.parametrize("fmt", [0, 1])
def test_single_linear_weight(fp4w, fmt):
    w, _, _, _ = W.linear_inputs(0, 256, 512, 1)
    _compare(fp4w, w, fmt, "single linear 256x512 seed 0")


@pytest.mark.parametrize("fmt", [0, 1])
def test_full_size_gate_up(fp4w, fmt):
    shape = W.QWEN7B_SHAPES["gate_up"]
    w = W.outlier_weights(3, 0, shape) if fmt == 0 else W.student_t_weights(3, 0, shape)
    _compare(fp4w, w, fmt, f"Qwen-2.5-7B gate/up {shape}")


@pytest.mark.parametrize("fmt", [0, 1])
def test_ragged_and_activation_shapes(fp4w, fmt):
    # rows not a multiple of anything, K = 32 (one MXFP4 block), and an activation-shaped x
    rng = np.random.default_rng(21)
    for (n, k) in [(7, 32), (33, 96), (1, 3584), (64, 2048)]:
        w = W.to_bf16_bits(rng.standard_normal((n, k)))
        _compare(fp4w, w, fmt, f"({n}, {k})")


@pytest.mark.parametrize("fmt", [0, 1])
def test_special_values(fp4w, fmt):
    rng = np.random.default_rng(11)
    vals = rng.standard_normal((8, 256)) * 0.02
    vals[1] = 0.0
    vals[3, :64] = 2.0 ** -130 * rng.integers(1, 8, 64)   # bf16 subnormals
    vals[4, :32] = 3.0e38 * rng.choice([-1, 1], 32)       # near the bf16 maximum (MXFP4 scale 0xFD/0xFE)
    vals[5, 16:32] = 1.0e-12
    vals[6] = rng.standard_normal(256) * 1e-30
    bits = W.to_bf16_bits(vals)
    bits[2, :32] = 0x8000                                 # -0
    _compare(fp4w, bits, fmt, "special values")


@pytest.mark.parametrize("fmt", [0, 1])
def test_tiny_tensors(fp4w, fmt):
    rng = np.random.default_rng(12)
    _compare(fp4w, W.to_bf16_bits(rng.standard_normal((4, 64)) * 1e-22), fmt, "tiny tensor")
    _compare(fp4w, W.to_bf16_bits(rng.standard_normal((4, 64)) * 2.0 ** -128), fmt, "subnormal tensor")


def test_nonfinite_mxfp4_block(fp4w):
    # an inf in a block: NaN scale 0xFF, the whole block decodes to NaN, other blocks unaffected
    w = W.to_bf16_bits(np.ones((2, 64)))
    w[1, 7] = 0x7F80
    _compare(fp4w, w, 1, "inf in one MXFP4 block")


@pytest.mark.parametrize("fmt", [0, 1])
def test_frozen_scales(fp4w, fmt):
    say(f"[fake-quant] frozen fmt={fmt}")
    w = W.outlier_weights(7, 0, (300, 1024), p=0.01)
    rng = np.random.default_rng(8)
    nb = 1024 // (16 if fmt == 0 else 32)
    scales = rng.integers(0, 0x7F, (300, nb)).astype(np.uint8) if fmt == 0 else \
        rng.integers(100, 140, (300, nb)).astype(np.uint8)
    st = np.float32(3.7e-5)
    frozen = fp4w.QWeight(fmt, None, u8_dev(scales), f32_dev([st]) if fmt == 0 else None, 300, 1024)
    y, s_out, _ = fp4w.fake_quant(bf16_dev(w), fmt, frozen=frozen)
    torch.cuda.synchronize()
    codes = O.quantize_frozen(fmt, w, scales, st)
    want = O.dequantize(fmt, codes, scales, st, "bf16")
    got = bits_host(y)
    assert np.array_equal(got, want), f"{np.sum(got != want)} values differ"
    assert np.array_equal(s_out.cpu().numpy(), scales)              # scales untouched


@pytest.mark.parametrize("fmt", [0, 1])
def test_matches_quantize_then_dequantize_on_device(fp4w, fmt):
    """The fused pass equals the library's own two-step path (quantize, then
    dequantize) on the same tensor."""
    w = bf16_dev(W.outlier_weights(9, 0, (512, 2048)))
    y, _, _ = fp4w.fake_quant(w, fmt)
    y2 = fp4w.dequantize(fp4w.quantize(w, fmt), torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


def test_straight_through_backward(fp4w):
    w = torch.randn(64, 256, device=DEV).to(torch.bfloat16).requires_grad_(True)
    y = fp4w.FakeQuantSTE.apply(w, 0)
    g = torch.randn_like(y)
    y.backward(g)
    assert torch.equal(w.grad.view(torch.int16), g.view(torch.int16))
    y_ref, _, _ = fp4w.fake_quant(w.detach(), 0)
    assert torch.equal(y.detach().view(torch.int16), y_ref.view(torch.int16))
