"""GPU parity of the Scale-QLoRA delta gradient (fp4w_scale_delta_grad) against
the binary64 oracle, within |err| <= 2e-3 ||dY[:, n]|| sum_{k in b} s_t |e2m1(q)| ||X[:, k]||.

Weights quantized by the oracle on the CPU, x and dY ~ N(0, 1); ragged shapes
against the full oracle, the gate/up layer at 2048 tokens on sampled blocks."""
import numpy as np
import pytest
import torch

import oracle as O
from mxfp4_bit_weight_amd import workloads as W
from tests.gpu_util import DEV, Guarded, bf16_dev, check_bound, f64_of_bf16, qweight_dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp4w():
    from mxfp4_bit_weight_amd import fp4w as F
    return F


def _bound_terms(fmt, dy, x, codes, st, rows=None, blocks=None):
    blk = O.BLOCK[fmt]
    n, k = codes.shape[0], codes.shape[1] * 2
    unit = np.full((n, k // blk), 0x38 if fmt == 0 else 127, np.uint8)
    e = np.abs(O.dequantize(fmt, codes, unit, 1.0, "f64")) * (float(np.float32(st)) if fmt == 0 else 1.0)
    xn = np.sqrt((f64_of_bf16(x) ** 2).sum(axis=0))                  # ||X[:, k]||
    yn = np.sqrt((f64_of_bf16(dy) ** 2).sum(axis=0))                 # ||dY[:, n]||
    wsum = (e * xn[None, :]).reshape(n, k // blk, blk).sum(axis=2)  # sum_k |c| ||X_k||
    if rows is None:
        return yn[:, None], wsum
    return yn[rows], wsum[rows, blocks]


SHAPES = [(257, 304, 256), (600, 520, 1280), (33, 1032, 512), (300, 264, 96), (1, 8, 32), (130, 72, 4128),
          (64, 128, 128), (0, 16, 64)]


@pytest.mark.parametrize("m,n,k", SHAPES)
@pytest.mark.parametrize("fmt", [0, 1])
def test_delta_grad_ragged(fp4w, fmt, m, n, k):
    say(f"[delta-grad] fmt={fmt} m={m} n={n} k={k}")
    w = W.outlier_weights(m + n, 0, (n, k)) if fmt == 0 else W.student_t_weights(m + n, 0, (n, k))
    codes, scales, st = O.quantize(fmt, w)
    rng = np.random.default_rng(m * 3 + k)
    dy = W.to_bf16_bits(rng.standard_normal((m, n)))
    x = W.to_bf16_bits(rng.standard_normal((m, k)))
    guard = Guarded(scales.shape, torch.float32, float("nan"))
    g = fp4w.scale_delta_grad(bf16_dev(dy).view(m, n), bf16_dev(x).view(m, k),
                              qweight_dev(fp4w, fmt, codes, scales, st), out=guard.t)
    guard.check(f"delta grad fmt={fmt} m={m} n={n} k={k}")
    want = O.scale_delta_grad(fmt, dy.reshape(m, n), x.reshape(m, k), codes, st)
    yn, ws = _bound_terms(fmt, dy.reshape(m, n), x.reshape(m, k), codes, st)
    check_bound(g.cpu().numpy().astype(np.float64), want, yn, ws, f"fmt={fmt} m={m} n={n} k={k}")


@pytest.mark.parametrize("fmt", [0, 1])
def test_delta_grad_gate_up_sampled(fp4w, fmt):
    m, (n, k) = 2048, W.QWEN7B_SHAPES["gate_up"]
    say(f"[delta-grad] gate/up fmt={fmt} m={m} n={n} k={k} (sampled)")
    w = W.outlier_weights(41, 0, (n, k)) if fmt == 0 else W.student_t_weights(41, 0, (n, k))
    codes, scales, st = O.quantize(fmt, w)
    rng = np.random.default_rng(42)
    dy = W.to_bf16_bits(rng.standard_normal((m, n)) * 0.01)
    x = W.to_bf16_bits(rng.standard_normal((m, k)))
    g = fp4w.scale_delta_grad(bf16_dev(dy), bf16_dev(x), qweight_dev(fp4w, fmt, codes, scales, st))
    torch.cuda.synchronize()
    blk = O.BLOCK[fmt]
    rows, blocks = rng.integers(0, n, 512), rng.integers(0, k // blk, 512)
    got = g.cpu().numpy()[rows, blocks].astype(np.float64)
    cols = (blocks[:, None] * blk + np.arange(blk)[None, :])                       # (s, blk)
    gmat = np.einsum("ms,msb->sb", f64_of_bf16(dy[:, rows]), f64_of_bf16(x[:, cols.reshape(-1)]).reshape(m, -1, blk))
    unit = np.full((512, k // blk), 0x38 if fmt == 0 else 127, np.uint8)
    e2m1 = O.dequantize(fmt, codes[rows], unit, 1.0, "f64")[np.arange(512)[:, None], cols]
    ts = float(np.float32(st)) if fmt == 0 else 1.0
    want = ts * (e2m1 * gmat).sum(axis=1)
    yn = np.sqrt((f64_of_bf16(dy[:, rows]) ** 2).sum(axis=0))
    xn = np.sqrt((f64_of_bf16(x[:, cols.reshape(-1)]) ** 2).sum(axis=0)).reshape(512, blk)
    check_bound(got, want, yn, ts * (np.abs(e2m1) * xn).sum(axis=1), f"gate/up delta grad fmt={fmt}")
