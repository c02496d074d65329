"""The LoRA branch of the W4A16 linear, pinned at the shapes that run it.

With every code zero the dequantized base is exactly 0 (0 times any finite
block scale), so the linear reduces to y = (x A^T) B^T = x (B A)^T (Telegram
post, "Metod": a LoRA adapter in parallel to the frozen 4-bit base).  The
acceptance bound then tightens to 2e-3 * ||x_m|| * ||(B A)[n]||, which is about
an eighth of a typical output at K = 3584: a dropped K chunk of the LoRA
down-projection, a wrong row of t or a missing LoRA epilogue fails it on most
outputs (a base-path output that leaked in would too).

Covered: the m = 1 block-scaled decode kernel with its in-launch hand-over of t
(default wait bound, and bound 0 where most workgroups form t themselves), the
m = 8 x-in-registers decode kernel, and the m = 16384 GEMM (t split into two
bf16 parts for the matrix core) on sampled outputs; the Qwen-2.5-7B gate/up
(18944, 3584) and down (3584, 18944) projections; ranks 16, 17 and 64; both
formats.  Outputs start as NaN, so every one must have been written.

A second, tighter check follows from the arithmetic of the branch: x, A and B
are exact bf16 values, t is accumulated in fp32 (or split into two bf16 parts,
2^-16 relative), so apart from fp32 summation error (far below 1e-4 relative)
the only sizable error is the final bf16 rounding of y (at most 2^-9 of |y|):
|err| <= 2^-8 |y64| + 1e-4 ||x_m|| ||(B A)[n]||."""
import numpy as np
import pytest
import torch

import oracle as O
from mxfp4_bit_weight_amd import workloads as W
from tests.gpu_util import DEV, bf16_dev, bits_host, check_bound, f64_of_bf16, qweight_dev, say

pytestmark = pytest.mark.gpu

SHAPES = {"gate_up": W.QWEN7B_SHAPES["gate_up"], "down": W.QWEN7B_SHAPES["down"]}


@pytest.fixture(scope="module")
def fp4w():
    from mxfp4_bit_weight_amd import fp4w as F
    return F


@pytest.fixture
def restore_wait(fp4w):
    prev = fp4w.debug_lora_wait()
    yield
    fp4w.debug_lora_wait(prev)


def _zero_code_weight(fmt, n, k, seed):
    """All-zero codes under valid, varied block scales (and an NVFP4 tensor scale)."""
    g = np.random.default_rng(seed)
    codes = np.zeros((n, k // 2), np.uint8)
    if fmt == 0:
        scales = g.integers(0x00, 0x7F, (n, k // 16)).astype(np.uint8)     # E4M3 0x00..0x7E
        st = np.float32(0.02 * 20 / 2688)
    else:
        scales = g.integers(100, 140, (n, k // 32)).astype(np.uint8)        # E8M0 2^-27 .. 2^12
        st = np.float32(1.0)
    return codes, scales, st


def _ba_norms(a, b):
    """||(B A)[n, :]||_2 in binary64 for every n, through the Gram matrix A A^T."""
    af, bf = f64_of_bf16(a), f64_of_bf16(b)
    gram = af @ af.T
    return np.sqrt(np.maximum(((bf @ gram) * bf).sum(axis=1), 0.0))


def _strict(yg, y64, xn, wn, what):
    err = np.abs(yg - y64)
    lim = 2.0 ** -8 * np.abs(y64) + 1e-4 * xn * wn
    bad = ~(err <= lim)
    assert not bad.any(), (f"{what}: {bad.sum()} outputs beyond the bf16-rounding bound; worst "
                           f"err={err[bad].max():.3e}")


def _lora_inputs(seed, n, k, m, r):
    _, x, a, b = W.linear_inputs(seed, n, k, m, rank=r)
    return x, a, b


def _decode_case(fp4w, fmt, name, m, r, wait0=False):
    n, k = SHAPES[name]
    what = f"zero codes fmt={fmt} {name} m={m} r={r}" + (" wait=0" if wait0 else "")
    say(f"[lora pinned] {what}")
    seed = 500 + 31 * r + m + (7 if name == "down" else 0)
    codes, scales, st = _zero_code_weight(fmt, n, k, seed)
    x, a, b = _lora_inputs(seed, n, k, m, r)
    q = qweight_dev(fp4w, fmt, codes, scales, st)
    ws = torch.zeros(fp4w.linear_workspace_bytes(m, n, k, r), dtype=torch.uint8, device=DEV)
    if wait0:
        fp4w.debug_lora_wait(0)
    y = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=DEV)
    fp4w.linear(bf16_dev(x), q, bf16_dev(a), bf16_dev(b), out=y, workspace=ws)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all().item()), "an output was not written"
    assert int(ws[:fp4w.WORKSPACE_COUNTER_BYTES].view(torch.int32).abs().sum().item()) == 0
    yg = f64_of_bf16(bits_host(y))
    y64 = O.linear(fmt, x, codes, scales, st, a, b)
    assert np.abs(y64).max() > 0
    xn = np.sqrt((f64_of_bf16(x) ** 2).sum(axis=1))[:, None]
    wn = _ba_norms(a, b)[None, :]
    check_bound(yg, y64, xn, wn, what)
    _strict(yg, y64, xn, wn, what)


@pytest.mark.parametrize("r", [16, 17, 64])
@pytest.mark.parametrize("name", ["gate_up", "down"])
@pytest.mark.parametrize("fmt", [0, 1])
def test_lora_m1_handover(fp4w, restore_wait, fmt, name, r):
    _decode_case(fp4w, fmt, name, 1, r)


@pytest.mark.parametrize("r", [16, 17, 64])
@pytest.mark.parametrize("name", ["gate_up", "down"])
@pytest.mark.parametrize("fmt", [0, 1])
def test_lora_m1_own_t(fp4w, restore_wait, fmt, name, r):
    _decode_case(fp4w, fmt, name, 1, r, wait0=True)


@pytest.mark.parametrize("r", [16, 17, 64])
@pytest.mark.parametrize("name", ["gate_up", "down"])
@pytest.mark.parametrize("fmt", [0, 1])
def test_lora_m8(fp4w, fmt, name, r):
    _decode_case(fp4w, fmt, name, 8, r)


_X_PREFILL = {}


def _prefill_x(k):
    if k not in _X_PREFILL:
        _X_PREFILL.clear()
        _X_PREFILL[k] = W.normal_bf16(900 + k, W.TID_X, (W.PREFILL_M, k), 1.0)
    return _X_PREFILL[k]


@pytest.mark.parametrize("name,r", [("gate_up", 16), ("gate_up", 17), ("gate_up", 64), ("down", 16)])
@pytest.mark.parametrize("fmt", [0, 1])
def test_lora_prefill_gemm(fp4w, fmt, name, r):
    """m = 16384 (batch 8 x 2048): 4096 sampled outputs, every output written."""
    n, k = SHAPES[name]
    m = W.PREFILL_M
    what = f"zero codes fmt={fmt} {name} m={m} r={r}"
    say(f"[lora pinned] {what}")
    seed = 700 + r + (7 if name == "down" else 0)
    codes, scales, st = _zero_code_weight(fmt, n, k, seed)
    _, a, b = _lora_inputs(seed, n, k, 1, r)
    x = _prefill_x(k)
    q = qweight_dev(fp4w, fmt, codes, scales, st)
    y = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=DEV)
    fp4w.linear(bf16_dev(x), q, bf16_dev(a), bf16_dev(b), out=y)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all().item()), "an output was not written"
    rng = np.random.default_rng(seed)
    rows = rng.integers(0, m, 4096)
    cols = rng.integers(0, n, 4096)
    yg = f64_of_bf16(bits_host(y[torch.from_numpy(rows).to(DEV), torch.from_numpy(cols).to(DEV)]))
    del y
    y64 = O.linear_sampled(fmt, x, codes, scales, st, rows, cols, a, b)
    xn = np.sqrt((f64_of_bf16(x[rows]) ** 2).sum(axis=1))
    wn = _ba_norms(a, b)[cols]
    check_bound(yg, y64, xn, wn, what)
    _strict(yg, y64, xn, wn, what)
