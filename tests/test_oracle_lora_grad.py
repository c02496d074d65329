"""Pins of the LoRA-gradient oracle (oracle.lora_backward) against the forward
oracle in C (oracle.linear), which it shares no code with.

The LoRA branch y_lora = (x A^T) B^T is linear in each of x, A and B, so for any
direction E the derivative of <dY, y_lora> along E equals <dY, y_lora with that
argument replaced by E>.  With all-zero codes the C forward computes exactly
y_lora, so each gradient is checked against it along random bf16 directions and
along the argument itself (<dB, B> = <dA, A> = <dX_lora, x> = <dY, y_lora>):
a transposed operand, a dropped factor or a wrong index fails these.  t and u
are pinned by one-hot rows of x and dY."""
import numpy as np
import pytest

import oracle as O
from mxfp4_bit_weight_amd import workloads as W


def f64(b):
    return W.bf16_bits_to_f32(b).astype(np.float64)


def _forward(x, a, b, n, k):
    """y_lora from the C forward oracle: zero codes (NVFP4, unit scales)."""
    codes = np.zeros((n, k // 2), np.uint8)
    scales = np.full((n, k // 16), 0x38, np.uint8)
    return O.linear(O.NVFP4, x, codes, scales, np.float32(1.0), a, b)


@pytest.mark.parametrize("m,n,k,r", [(3, 40, 64, 16), (5, 17 * 2, 96, 5), (1, 16, 32, 1), (7, 48, 128, 33)])
def test_gradients_are_adjoints_of_the_forward(m, n, k, r):
    rng = np.random.default_rng(m * 100 + r)
    _, x, a, b = W.linear_inputs(11 + m, n, k, m, rank=r)
    dy = W.to_bf16_bits(rng.standard_normal((m, n)))
    t, u, da, db, dx = O.lora_backward(dy, x, a, b)
    base = float((f64(dy) * _forward(x, a, b, n, k)).sum())
    scale = abs(base) + float(np.abs(f64(dy)).sum() * np.abs(_forward(x, a, b, n, k)).max()) * 1e-12 + 1e-300
    # along the arguments themselves
    for g, arg in ((db, b), (da, a), (dx, x)):
        assert abs(float((g * f64(arg)).sum()) - base) <= 1e-10 * scale
    # along random directions
    eb = W.to_bf16_bits(rng.standard_normal((n, r)))
    ea = W.to_bf16_bits(rng.standard_normal((r, k)))
    ex = W.to_bf16_bits(rng.standard_normal((m, k)))
    for g, d, y_dir in ((db, eb, _forward(x, a, eb, n, k)), (da, ea, _forward(x, ea, b, n, k)),
                        (dx, ex, _forward(ex, a, b, n, k))):
        want = float((f64(dy) * y_dir).sum())
        got = float((g * f64(d)).sum())
        assert abs(got - want) <= 1e-9 * (np.abs(f64(dy)).sum() * np.abs(y_dir).max() + 1e-300)


def test_t_and_u_one_hot():
    m, n, k, r = 4, 32, 64, 16
    _, x, a, b = W.linear_inputs(3, n, k, m, rank=r)
    one = W.to_bf16_bits(np.eye(m, k))             # x row i = e_i: t row i = column i of A
    dy = W.to_bf16_bits(np.eye(m, n) * 2.0)        # dY row i = 2 e_i: u row i = 2 B[i]
    t, u, _, _, _ = O.lora_backward(dy, one, a, b)
    assert np.array_equal(t, f64(a)[:, :m].T)
    assert np.array_equal(u, 2.0 * f64(b)[:m])
