"""GPU parity of the input gradient through the frozen base
(fp4w_linear_backward_dx): dX = dY deq(W) against the binary64 oracle, within
|err| <= 2e-3 ||dY_m|| ||deq(W)[:, k]||.

Weights are quantized by the oracle on the CPU (NVFP4 with outliers, MXFP4
heavy-tailed), dY ~ N(0, 1); ragged shapes run against the full oracle, the
gate/up backward shape on sampled outputs."""
import numpy as np
import pytest
import torch

import oracle as O
from mxfp4_bit_weight_amd import workloads as W
from tests.gpu_util import DEV, Guarded, bf16_dev, bits_host, check_bound, f64_of_bf16, qweight_dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp4w():
    from mxfp4_bit_weight_amd import fp4w as F
    return F


def _weights(fmt, seed, n, k):
    w = W.outlier_weights(seed, 0, (n, k)) if fmt == 0 else W.student_t_weights(seed, 0, (n, k))
    return O.quantize(fmt, w)


def _col_norms(fmt, codes, scales, st, cols=None):
    d = O.dequantize(fmt, codes, scales, st, "f64")
    if cols is not None:
        d = d[:, cols]
    return np.sqrt((d * d).sum(axis=0))


SHAPES = [(257, 304, 256), (600, 520, 1280), (33, 1032, 512), (300, 264, 96), (1, 8, 32), (130, 72, 4128),
          (128, 64, 128)]


@pytest.mark.parametrize("m,n,k", SHAPES)
@pytest.mark.parametrize("fmt", [0, 1])
def test_backward_dx_ragged(fp4w, fmt, m, n, k):
    say(f"[backward] fmt={fmt} m={m} n={n} k={k}")
    codes, scales, st = _weights(fmt, m + n + k, n, k)
    rng = np.random.default_rng(m * 7 + n)
    dy = W.to_bf16_bits(rng.standard_normal((m, n)))
    q = qweight_dev(fp4w, fmt, codes, scales, st)
    g = Guarded((m, k), torch.bfloat16, float("nan"))
    dx = fp4w.linear_backward_dx(bf16_dev(dy), q, out=g.t)
    g.check(f"backward dx fmt={fmt} m={m} n={n} k={k}")
    want = O.linear_backward_dx(fmt, dy, codes, scales, st)
    yn = np.sqrt((f64_of_bf16(dy) ** 2).sum(axis=1))[:, None]
    check_bound(f64_of_bf16(bits_host(dx)), want, yn, _col_norms(fmt, codes, scales, st)[None, :],
                f"fmt={fmt} m={m} n={n} k={k}")


@pytest.mark.parametrize("fmt", [0, 1])
def test_backward_dx_nan_scale_and_empty_n(fp4w, fmt):
    m, n, k = 40, 48, 128
    codes, scales, st = _weights(fmt, 3, n, k)
    scales = scales.copy()
    blk = 16 if fmt == 0 else 32
    scales[7, 1] = 0x7F if fmt == 0 else 0xFF          # NaN scale: block 1 of row 7
    dy = W.to_bf16_bits(np.random.default_rng(4).standard_normal((m, n)))
    dx = f64_of_bf16(bits_host(fp4w.linear_backward_dx(bf16_dev(dy), qweight_dev(fp4w, fmt, codes, scales, st))))
    torch.cuda.synchronize()
    nan_cols = np.zeros(k, bool)
    nan_cols[blk:2 * blk] = True
    assert np.isnan(dx[:, nan_cols]).all()
    assert not np.isnan(dx[:, ~nan_cols]).any()
    # n == 0: dx = 0
    q0 = fp4w.QWeight(fmt, torch.empty((0, k // 2), dtype=torch.uint8, device=DEV),
                      torch.empty((0, k // blk), dtype=torch.uint8, device=DEV),
                      torch.ones(1, dtype=torch.float32, device=DEV) if fmt == 0 else None, 0, k)
    out = torch.full((5, k), float("nan"), dtype=torch.bfloat16, device=DEV)
    fp4w.linear_backward_dx(torch.empty((5, 0), dtype=torch.bfloat16, device=DEV), q0, out=out)
    torch.cuda.synchronize()
    assert not out.float().any().item()


@pytest.mark.parametrize("fmt", [0, 1])
def test_backward_dx_gate_up_sampled(fp4w, fmt):
    # backward of the Qwen-2.5-7B gate/up linear (W 18944 x 3584) for 2048 tokens
    m, (n, k) = 2048, W.QWEN7B_SHAPES["gate_up"]
    say(f"[backward] gate/up fmt={fmt} m={m} n={n} k={k} (sampled)")
    codes, scales, st = _weights(fmt, 31, n, k)
    rng = np.random.default_rng(32)
    dy = W.to_bf16_bits(rng.standard_normal((m, n)) * 0.01)
    dx = fp4w.linear_backward_dx(bf16_dev(dy), qweight_dev(fp4w, fmt, codes, scales, st))
    torch.cuda.synchronize()
    rows, cols = rng.integers(0, m, 2048), rng.integers(0, k, 2048)
    got = f64_of_bf16(bits_host(dx[torch.from_numpy(rows).to(DEV), torch.from_numpy(cols).to(DEV)]))
    deq = O.dequantize(fmt, codes, scales, st, "f64")
    dyf = f64_of_bf16(dy[rows])
    want = np.einsum("sn,ns->s", dyf, deq[:, cols])
    check_bound(got, want, np.sqrt((dyf ** 2).sum(axis=1)), np.sqrt((deq[:, cols] ** 2).sum(axis=0)),
                f"gate/up backward fmt={fmt}")
