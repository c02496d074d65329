"""GPU parity of the LoRA gradients (fp4w_lora_backward: u = dY B, dA = u^T x,
dB = dY^T (x A^T)) and of the adapter's term u A in the input gradient
(fp4w_linear_backward_dx), against the binary64 oracle (oracle.lora_backward).

Bounds, in the style of the linear's (each output against the norms of the two
vectors it contracts):
    |u - u64|[m, j]   <= 2e-3 ||dY[m, :]|| ||B[:, j]||
    |dB - dB64|[n, j] <= 2e-3 ||dY[:, n]|| ||t64[:, j]||
    |dA - dA64|[j, k] <= 2e-3 ||u64[:, j]|| ||x[:, k]||
    |dX - dX64|[m, k] <= 2e-3 ||dY[m, :]|| ||(deq(W) + B A)[:, k]|| + 2^-8 |dX64|
(the last term: the one bf16 rounding of dX, which a short contraction makes
comparable to the first)
and a tighter one the arithmetic gives (fp32 sums, t and u as two bf16 parts,
2^-16 relative): the same with 1e-4 (dX: plus half a bf16 ulp of the result).
Shapes: ragged m, n, k and ranks 1, 5, 16, 17, 64 over several tiles and splits;
m = 0 (zero gradients, outputs pre-filled with NaN); the Qwen-2.5-7B gate/up
layer at 2048 tokens on sampled outputs."""
import numpy as np
import pytest
import torch

import oracle as O
from mxfp4_bit_weight_amd import workloads as W
from tests.gpu_util import DEV, Guarded, bf16_dev, bits_host, check_bound, f32_dev, f64_of_bf16, qweight_dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp4w():
    from mxfp4_bit_weight_amd import fp4w as F
    return F


def _inputs(seed, m, n, k, r):
    _, x, a, b = W.linear_inputs(seed, n, k, m, rank=r)
    dy = W.normal_bf16(seed, W.TID_DELTA + 10, (m, n), 1.0)
    return dy, x, a, b


def _both(got, want, xn, wn, what):
    check_bound(got, want, xn, wn, what)
    err = np.abs(got - want)
    lim = 1e-4 * xn * wn
    assert (err <= lim).all(), f"{what}: beyond the fp32 bound, worst {float((err / np.maximum(lim, 1e-300)).max()):.2f}x"


def _check_grads(fmt_what, dy, x, a, b, u, ga, gb):
    t64, u64, da64, db64, _ = O.lora_backward(dy, x, a, b)
    dyf, xf, af, bf = f64_of_bf16(dy), f64_of_bf16(x), f64_of_bf16(a), f64_of_bf16(b)
    _both(u, u64, np.linalg.norm(dyf, axis=1)[:, None], np.linalg.norm(bf, axis=0)[None, :], f"u {fmt_what}")
    _both(gb, db64, np.linalg.norm(dyf, axis=0)[:, None], np.linalg.norm(t64, axis=0)[None, :], f"dB {fmt_what}")
    _both(ga, da64, np.linalg.norm(u64, axis=0)[:, None], np.linalg.norm(xf, axis=0)[None, :], f"dA {fmt_what}")


RAGGED = [(1, 8, 32, 1), (37, 104, 96, 16), (300, 264, 544, 17), (64, 48, 128, 64), (513, 1032, 1056, 16),
          (70, 8, 4128, 5)]


@pytest.mark.parametrize("m,n,k,r", RAGGED)
def test_lora_gradients_ragged(fp4w, m, n, k, r):
    what = f"m={m} n={n} k={k} r={r}"
    say(f"[lora grad] {what}")
    dy, x, a, b = _inputs(m + 3 * r, m, n, k, r)
    guards = [Guarded((m, r), torch.float32, float("nan")), Guarded((r, k), torch.float32, float("nan")),
              Guarded((n, r), torch.float32, float("nan"))]
    u, ga, gb = fp4w.lora_backward(bf16_dev(dy), bf16_dev(x), bf16_dev(a), bf16_dev(b),
                                   out=tuple(g.t for g in guards))
    for g in guards:
        g.check(f"lora grads {what}")
    _check_grads(what, dy, x, a, b, u.double().cpu().numpy(), ga.double().cpu().numpy(), gb.double().cpu().numpy())
    # the same call again: bit for bit (every sum in a fixed order)
    u2, ga2, gb2 = fp4w.lora_backward(bf16_dev(dy), bf16_dev(x), bf16_dev(a), bf16_dev(b))
    torch.cuda.synchronize()
    for p, q in ((u, u2), (ga, ga2), (gb, gb2)):
        assert torch.equal(p.view(torch.int32), q.view(torch.int32))


def test_lora_gradients_zero_rows(fp4w):
    """m = 0: dA and dB are zero (written over NaN), u is empty."""
    n, k, r = 40, 64, 16
    _, _, a, b = W.linear_inputs(5, n, k, 1, rank=r)
    dy = torch.empty((0, n), dtype=torch.bfloat16, device=DEV)
    x = torch.empty((0, k), dtype=torch.bfloat16, device=DEV)
    ga = torch.full((r, k), float("nan"), device=DEV)
    gb = torch.full((n, r), float("nan"), device=DEV)
    ws = torch.empty(fp4w.lora_backward_workspace_bytes(0, n, k, r), dtype=torch.uint8, device=DEV)
    fp4w._check(fp4w._lora_bwd(fp4w._ptr(dy), 0, n, fp4w._ptr(x), k, fp4w._ptr(bf16_dev(a)), fp4w._ptr(bf16_dev(b)), r,
                               None, fp4w._ptr(ga), fp4w._ptr(gb), fp4w._ptr(ws), ws.numel(), fp4w._stream(DEV)), "m=0")
    torch.cuda.synchronize()
    assert bool((ga == 0).all().item()) and bool((gb == 0).all().item())


DX_CASES = [(37, 104, 96, 16), (300, 264, 544, 17), (130, 1032, 1056, 64), (64, 8, 4128, 1)]


@pytest.mark.parametrize("m,n,k,r", DX_CASES)
@pytest.mark.parametrize("fmt", [0, 1])
def test_backward_dx_with_lora_term(fp4w, fmt, m, n, k, r):
    """dX = dY deq(W) + u A with u from the oracle (the kernel's own term) and
    with u from fp4w_lora_backward (the chain a training step runs)."""
    what = f"fmt={fmt} m={m} n={n} k={k} r={r}"
    say(f"[lora dx] {what}")
    dy, x, a, b = _inputs(7 * m + r, m, n, k, r)
    w = W.weights("outlier" if fmt == 0 else "student_t", 7 * m + r, W.TID_W, (n, k))
    codes, scales, st = O.quantize(fmt, w)
    q = qweight_dev(fp4w, fmt, codes, scales, st)
    _, u64, _, _, dxl64 = O.lora_backward(dy, x, a, b)
    dx64 = O.linear_backward_dx(fmt, dy, codes, scales, st) + dxl64
    deq = O.dequantize(fmt, codes, scales, st, "f64") + f64_of_bf16(b) @ f64_of_bf16(a)
    dn = np.linalg.norm(f64_of_bf16(dy), axis=1)[:, None]
    wn = np.linalg.norm(deq, axis=0)[None, :]
    for src in ("oracle u", "device u"):
        if src == "oracle u":
            ud = f32_dev(u64.astype(np.float32))
        else:
            ud, _, _ = fp4w.lora_backward(bf16_dev(dy), bf16_dev(x), bf16_dev(a), bf16_dev(b))
        out = torch.full((m, k), float("nan"), dtype=torch.bfloat16, device=DEV)
        fp4w.linear_backward_dx(bf16_dev(dy), q, out=out, lora_u=ud, lora_a=bf16_dev(a))
        torch.cuda.synchronize()
        got = f64_of_bf16(bits_host(out))
        # the arithmetic bound plus the one rounding of the result to bf16 (at most
        # 2^-8 of it): with a short contraction (n = 8) |dX| can come within a factor
        # 2 of ||dY_m|| ||w_k||, where that rounding alone exceeds 2e-3 ||dY_m|| ||w_k||
        err = np.abs(got - dx64)
        bad = ~(err <= 2e-3 * dn * wn + 2.0 ** -8 * np.abs(dx64))
        assert not bad.any(), f"dX {what} ({src}): {bad.sum()} outputs outside the bound"
        lim = 1e-4 * dn * wn + 2.0 ** -8 * np.abs(dx64)
        assert (err <= lim).all(), f"dX {what} ({src}): beyond the fp32 bound"


def test_backward_dx_lora_only_when_n_is_zero(fp4w):
    """n = 0: no base term, dX = u A exactly as the kernel forms it."""
    m, k, r = 40, 256, 16
    _, x, a, _ = W.linear_inputs(9, 16, k, m, rank=r)
    u = np.random.default_rng(9).standard_normal((m, r)).astype(np.float32)
    q = fp4w.QWeight(0, torch.empty((0, k // 2), dtype=torch.uint8, device=DEV),
                     torch.empty((0, k // 16), dtype=torch.uint8, device=DEV), f32_dev([1.0]), 0, k)
    out = torch.full((m, k), float("nan"), dtype=torch.bfloat16, device=DEV)
    fp4w.linear_backward_dx(torch.empty((m, 0), dtype=torch.bfloat16, device=DEV), q, out=out, lora_u=f32_dev(u),
                            lora_a=bf16_dev(a))
    torch.cuda.synchronize()
    want = u.astype(np.float64) @ f64_of_bf16(a)
    got = f64_of_bf16(bits_host(out))
    lim = 1e-4 * np.linalg.norm(u, axis=1)[:, None] * np.linalg.norm(f64_of_bf16(a), axis=0)[None, :] \
        + 2.0 ** -8 * np.abs(want)
    assert (np.abs(got - want) <= lim).all()


def test_lora_gradients_gate_up_2048_tokens(fp4w):
    """The Qwen-2.5-7B gate/up layer (n 18944, k 3584, r 16) at 2048 tokens:
    every output written (NaN prefill), 2048 sampled outputs of each gradient."""
    m, (n, k), r = 2048, W.QWEN7B_SHAPES["gate_up"], 16
    say(f"[lora grad] gate/up m={m}")
    dy, x, a, b = _inputs(77, m, n, k, r)
    u, ga, gb = fp4w.lora_backward(bf16_dev(dy), bf16_dev(x), bf16_dev(a), bf16_dev(b))
    torch.cuda.synchronize()
    for tname, t_ in (("u", u), ("dA", ga), ("dB", gb)):
        assert bool(torch.isfinite(t_).all().item()), f"{tname}: an output was not written"
    t64, u64, da64, db64, _ = O.lora_backward(dy, x, a, b)
    dyf, xf, bf = f64_of_bf16(dy), f64_of_bf16(x), f64_of_bf16(b)
    rng = np.random.default_rng(77)
    uh, gah, gbh = u.double().cpu().numpy(), ga.double().cpu().numpy(), gb.double().cpu().numpy()
    mi, ji = rng.integers(0, m, 2048), rng.integers(0, r, 2048)
    _both(uh[mi, ji], u64[mi, ji], np.linalg.norm(dyf[mi], axis=1), np.linalg.norm(bf[:, ji], axis=0), "u sampled")
    ni = rng.integers(0, n, 2048)
    _both(gbh[ni, ji], db64[ni, ji], np.linalg.norm(dyf[:, ni], axis=0), np.linalg.norm(t64[:, ji], axis=0),
          "dB sampled")
    ki = rng.integers(0, k, 2048)
    _both(gah[ji, ki], da64[ji, ki], np.linalg.norm(u64[:, ji], axis=0), np.linalg.norm(xf[:, ki], axis=0),
          "dA sampled")
