"""GPU parity of the W4A4 MXFP4 GEMM (fp4w_linear_w4a4) against the binary64
oracle deq(x) deq(W)^T, within |err| <= 2e-3 ||deq(x)_m|| ||deq(W)_n||.

x and W are quantized to MXFP4 by the oracle on the CPU (activations ~ N(0, 1),
weights heavy-tailed), so the GEMM is checked on its own; ragged shapes run
against the full oracle, the full-size prefill shape and a many-tile grid on
sampled outputs."""
import numpy as np
import pytest
import torch

import oracle as O
from mxfp4_bit_weight_amd import workloads as W
from tests.gpu_util import DEV, Guarded, bf16_dev, bits_host, check_bound, f64_of_bf16, say, u8_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp4w():
    from mxfp4_bit_weight_amd import fp4w as F
    return F


def _q_dev(fp4w, codes, scales):
    n, kh = codes.shape
    return fp4w.QWeight(O.MXFP4, u8_dev(codes), u8_dev(scales), None, n, kh * 2)


def _norms(codes, scales, rows=None):
    if rows is not None:
        codes, scales = codes[rows], scales[rows]
    d = O.dequantize(O.MXFP4, codes, scales, 1.0, "f64")
    return np.sqrt((d * d).sum(axis=1))


def _inputs(seed, m, n, k):
    rng = np.random.default_rng(seed)
    x = W.to_bf16_bits(rng.standard_normal((m, k)))
    w = W.student_t_weights(seed, 0, (n, k))
    xc, xs, _ = O.quantize(O.MXFP4, x)
    wc, ws, _ = O.quantize(O.MXFP4, w)
    return xc, xs, wc, ws


def _full(fp4w, xc, xs, wc, ws, what):
    g = Guarded((xc.shape[0], wc.shape[0]), torch.bfloat16, float("nan"))
    y = fp4w.linear_w4a4(_q_dev(fp4w, xc, xs), _q_dev(fp4w, wc, ws), out=g.t)
    g.check(f"w4a4 {what}")
    yg = f64_of_bf16(bits_host(y))
    y64 = O.linear_w4a4(xc, xs, wc, ws)
    return check_bound(yg, y64, _norms(xc, xs)[:, None], _norms(wc, ws)[None, :], what)


SHAPES = [(257, 301, 256), (600, 520, 1280), (33, 1030, 512), (300, 257, 768), (40, 64, 128), (1, 1, 128),
          (256, 256, 128), (513, 17, 384)]


@pytest.mark.parametrize("m,n,k", SHAPES)
def test_w4a4_ragged(fp4w, m, n, k):
    say(f"[w4a4] m={m} n={n} k={k}")
    worst = _full(fp4w, *_inputs(m + n + k, m, n, k), f"m={m} n={n} k={k}")
    say(f"  worst relative error {worst:.2e}")


def test_w4a4_unaligned_y_and_odd_n(fp4w):
    # n odd: the 2-byte store path; y a view at an odd bf16 offset
    m, n, k = 70, 99, 256
    xc, xs, wc, ws = _inputs(5, m, n, k)
    buf = torch.full((m * n + 1,), float("nan"), dtype=torch.bfloat16, device=DEV)
    y = buf[1:].view(m, n)
    fp4w.linear_w4a4(_q_dev(fp4w, xc, xs), _q_dev(fp4w, wc, ws), out=y)
    torch.cuda.synchronize()
    assert torch.isnan(buf[0]).item()
    check_bound(f64_of_bf16(bits_host(y.contiguous())), O.linear_w4a4(xc, xs, wc, ws),
                _norms(xc, xs)[:, None], _norms(wc, ws)[None, :], "odd n, unaligned y")


def test_w4a4_scale_extremes(fp4w):
    # random code bytes under scales spread over 2^-60 .. 2^60 for x and W: the
    # products' exponents add; every output stays far inside fp32
    rng = np.random.default_rng(9)
    m, n, k = 64, 96, 512
    xc = rng.integers(0, 256, (m, k // 2)).astype(np.uint8)
    wc = rng.integers(0, 256, (n, k // 2)).astype(np.uint8)
    xs = rng.integers(67, 188, (m, k // 32)).astype(np.uint8)
    ws = rng.integers(67, 188, (n, k // 32)).astype(np.uint8)
    _full(fp4w, xc, xs, wc, ws, "scale extremes")


def test_w4a4_nan_scale(fp4w):
    # E8M0 0xFF is NaN: the outputs of that x row are NaN, the others unaffected
    m, n, k = 40, 48, 256
    xc, xs, wc, ws = _inputs(6, m, n, k)
    xs = xs.copy()
    xs[3, 2] = 0xFF
    y = fp4w.linear_w4a4(_q_dev(fp4w, xc, xs), _q_dev(fp4w, wc, ws))
    torch.cuda.synchronize()
    yg = f64_of_bf16(bits_host(y))
    assert np.isnan(yg[3]).all()
    keep = np.arange(m) != 3
    xs_ok = xs.copy()
    xs_ok[3, 2] = 127
    check_bound(yg[keep], O.linear_w4a4(xc, xs_ok, wc, ws)[keep], _norms(xc, xs_ok)[keep][:, None],
                _norms(wc, ws)[None, :], "rows without the NaN scale")


def test_w4a4_from_bf16_activations(fp4w):
    # the forward from bf16 x: quantized on the device, then the GEMM
    m, n, k = 300, 200, 512
    rng = np.random.default_rng(12)
    x = W.to_bf16_bits(rng.standard_normal((m, k)))
    w = W.student_t_weights(12, 0, (n, k))
    wc, ws, _ = O.quantize(O.MXFP4, w)
    y = fp4w.linear_a4(bf16_dev(x), _q_dev(fp4w, wc, ws))
    torch.cuda.synchronize()
    xc, xs, _ = O.quantize(O.MXFP4, x)
    check_bound(f64_of_bf16(bits_host(y)), O.linear_w4a4(xc, xs, wc, ws), _norms(xc, xs)[:, None],
                _norms(wc, ws)[None, :], "bf16 activations")


def _sampled(fp4w, m, n, k, seed, what, samples=4096):
    say(f"[w4a4] {what} m={m} n={n} k={k} (sampled)")
    rng = np.random.default_rng(seed)
    # random code bytes (every E2M1 value, both signs) and scales around 2^0
    xc = rng.integers(0, 256, (m, k // 2), dtype=np.uint8)
    wc = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    xs = rng.integers(120, 135, (m, k // 32), dtype=np.uint8)
    ws = rng.integers(115, 130, (n, k // 32), dtype=np.uint8)
    y = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=DEV)
    fp4w.linear_w4a4(_q_dev(fp4w, xc, xs), _q_dev(fp4w, wc, ws), out=y)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all().item()), "an output was not written"
    rows, cols = rng.integers(0, m, samples), rng.integers(0, n, samples)
    ys = f64_of_bf16(bits_host(y[torch.from_numpy(rows).to(DEV), torch.from_numpy(cols).to(DEV)]))
    y64 = O.linear_w4a4_sampled(xc, xs, wc, ws, rows, cols)
    check_bound(ys, y64, _norms(xc, xs, rows), _norms(wc, ws, cols), what)


def test_w4a4_more_tiles_than_cus(fp4w):
    _sampled(fp4w, 17 * 256 - 40, 17 * 256 - 40, 384, 77, "many tiles")


def test_w4a4_full_size_prefill(fp4w):
    # Qwen-2.5-7B gate/up at 16384 tokens
    _sampled(fp4w, 16384, 18944, 3584, 78, "prefill gate/up")


def test_binding_rejects_wrong_output_shapes(fp4w):
    # a wrong-sized output or frozen-scale buffer is refused before any launch
    m, n, k = 64, 32, 256
    xc, xs, wc, ws = _inputs(3, m, n, k)
    xq, q = _q_dev(fp4w, xc, xs), _q_dev(fp4w, wc, ws)
    with pytest.raises(ValueError):
        fp4w.linear_w4a4(xq, q, out=torch.empty((m, n - 1), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError):
        fp4w.linear_backward_dx(torch.zeros((m, n), dtype=torch.bfloat16, device=DEV), q,
                                out=torch.empty((m - 1, k), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError):
        fp4w.scale_delta_grad(torch.zeros((m, n), dtype=torch.bfloat16, device=DEV),
                              torch.zeros((m, k), dtype=torch.bfloat16, device=DEV), q,
                              out=torch.empty((n, k // 16), dtype=torch.float32, device=DEV))
    w = torch.zeros((n, k), dtype=torch.bfloat16, device=DEV)
    bad = fp4w.QWeight(1, None, torch.zeros((n, k // 32 - 1), dtype=torch.uint8, device=DEV), None, n, k)
    with pytest.raises(ValueError):
        fp4w.quantize(w, 1, frozen=bad)
    with pytest.raises(ValueError):
        fp4w.fake_quant(w, 1, frozen=bad)
    torch.cuda.synchronize()
