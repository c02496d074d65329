"""Decode-shaped linear on the block-scaled kernel (m = 1; m = 2; m <= 4 on small
matrices) with a LoRA: inside the one decode launch, the first workgroups form
t = x A^T (one K chunk each) and hand it to the workgroups that write the
outputs through words of the workspace.

Checked here, against the binary64 oracle within |err| <= 2e-3 ||x|| ||w_n^eff||:
  - shapes with fewer tiles than reader groups, ragged and maximal ranks, one
    tile with a long K (fewer workgroups than chunks: wider chunks), and the
    Qwen-2.5-7B projections (sampled outputs);
  - the outputs are bit for bit the same when the writers form t themselves:
    the host sets the kernel's own wait bound to 0 (fp4w_debug_lora_wait), so
    most of them do not wait for the published t;
  - after every call the counter area of the workspace is zero again, in both
    modes, so the next call of any shape starts clean."""
import numpy as np
import pytest
import torch

import oracle as O
from mxfp4_bit_weight_amd import workloads as W
from tests.gpu_util import DEV, bf16_dev, bits_host, check_bound, f64_of_bf16, qweight_dev, say, weff_norms

pytestmark = pytest.mark.gpu

# (n, k, r, sampled): one tile; ragged rank 1; maximal rank; one tile with long K;
# gate/up (1184 tiles); down with rank 17 (two column blocks of A)
CASES = [(16, 64, 16, False), (200, 544, 1, False), (1000, 1056, 64, False), (16, 8192, 16, False),
         (18944, 3584, 16, True), (3584, 18944, 17, True)]


@pytest.fixture(scope="module")
def fp4w():
    from mxfp4_bit_weight_amd import fp4w as F
    return F


@pytest.fixture
def restore_wait(fp4w):
    prev = fp4w.debug_lora_wait()
    yield
    fp4w.debug_lora_wait(prev)


def _counters_zero(fp4w, ws):
    return int(ws[:fp4w.WORKSPACE_COUNTER_BYTES].view(torch.int32).abs().sum().item()) == 0


def _check(fmt, y, x, codes, scales, st, a, b, sampled, what):
    n = y.shape[1]
    if not sampled:
        y64 = O.linear(fmt, x, codes, scales, st, a, b)
        xn = np.sqrt((f64_of_bf16(x) ** 2).sum(axis=1))[:, None]
        wn = weff_norms(fmt, codes, scales, st, a, b)[None, :]
        check_bound(f64_of_bf16(bits_host(y)), y64, xn, wn, what)
        return
    rng = np.random.default_rng(n)
    cols = rng.integers(0, n, 512)
    rows = np.zeros_like(cols)
    ys = f64_of_bf16(bits_host(y[0, torch.from_numpy(cols).to(DEV)]))
    y64 = O.linear_sampled(fmt, x, codes, scales, st, rows, cols, a, b)
    xn = np.sqrt((f64_of_bf16(x[rows]) ** 2).sum(axis=1))
    wn = weff_norms(fmt, codes, scales, st, a, b, rows=cols)
    check_bound(ys, y64, xn, wn, what)


@pytest.mark.parametrize("n,k,r,sampled", CASES)
@pytest.mark.parametrize("fmt", [0, 1])
def test_handover_matches_oracle_and_own_t(fp4w, restore_wait, fmt, n, k, r, sampled):
    what = f"fmt={fmt} m=1 n={n} k={k} r={r}"
    say(f"[lora handover] {what}")
    wkind = "outlier" if fmt == 0 else "student_t"
    w, x, a, b = W.linear_inputs(300 + r, n, k, 1, rank=r, wkind=wkind)
    codes, scales, st = O.quantize(fmt, w)
    q = qweight_dev(fp4w, fmt, codes, scales, st)
    xd, ad, bd = bf16_dev(x), bf16_dev(a), bf16_dev(b)
    ws = torch.zeros(fp4w.linear_workspace_bytes(1, n, k, r), dtype=torch.uint8, device=DEV)
    y1 = fp4w.linear(xd, q, ad, bd, workspace=ws)
    torch.cuda.synchronize()
    assert _counters_zero(fp4w, ws), "hand-over words left non-zero"
    _check(fmt, y1, x, codes, scales, st, a, b, sampled, what)
    fp4w.debug_lora_wait(0)
    for rep in range(2):
        y2 = fp4w.linear(xd, q, ad, bd, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), f"own t differs ({what}, rep {rep})"
        assert _counters_zero(fp4w, ws), "hand-over words left non-zero (wait bound 0)"


# m = 2 to 4 on the block-scaled kernel (m = 2 always; m = 3, 4 on matrices of
# at most 2^24 weights): several rows of x per chunk word
MROWS = [(2, 200, 544, 16), (2, 3584, 18944, 16), (3, 1000, 1056, 64), (4, 33, 640, 17), (4, 3584, 3584, 16)]


@pytest.mark.parametrize("m,n,k,r", MROWS)
@pytest.mark.parametrize("fmt", [0, 1])
def test_handover_several_rows(fp4w, restore_wait, fmt, m, n, k, r):
    what = f"fmt={fmt} m={m} n={n} k={k} r={r}"
    say(f"[lora handover] {what}")
    w, x, a, b = W.linear_inputs(400 + m + r, n, k, m, rank=r, wkind="outlier")
    codes, scales, st = O.quantize(fmt, w)
    q = qweight_dev(fp4w, fmt, codes, scales, st)
    xd, ad, bd = bf16_dev(x), bf16_dev(a), bf16_dev(b)
    ws = torch.zeros(fp4w.linear_workspace_bytes(m, n, k, r), dtype=torch.uint8, device=DEV)
    y1 = fp4w.linear(xd, q, ad, bd, workspace=ws)
    torch.cuda.synchronize()
    assert _counters_zero(fp4w, ws)
    rng = np.random.default_rng(m * 1000 + n)
    rows = rng.integers(0, m, 384)
    cols = rng.integers(0, n, 384)
    ys = f64_of_bf16(bits_host(y1[torch.from_numpy(rows).to(DEV), torch.from_numpy(cols).to(DEV)]))
    y64 = O.linear_sampled(fmt, x, codes, scales, st, rows, cols, a, b)
    xn = np.sqrt((f64_of_bf16(x[rows]) ** 2).sum(axis=1))
    wn = weff_norms(fmt, codes, scales, st, a, b, rows=cols)
    check_bound(ys, y64, xn, wn, what)
    fp4w.debug_lora_wait(0)
    y2 = fp4w.linear(xd, q, ad, bd, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), f"own t differs ({what})"
    assert _counters_zero(fp4w, ws)


def test_handover_then_other_shapes_on_one_workspace(fp4w):
    """m = 1 calls with LoRA ranks 64, 16 and 1 interleaved with other paths on one
    workspace: each result within the bound, the counter area zero after each."""
    say("[lora handover] interleaved shapes")
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device=DEV)
    for (m, n, k, r) in [(1, 1000, 1056, 64), (8, 1000, 2080, 16), (1, 16, 64, 16), (40, 300, 1056, 16),
                         (1, 200, 544, 1), (3, 1000, 1056, 64), (1, 1000, 1056, 64)]:
        w, x, a, b = W.linear_inputs(m * 13 + r, n, k, m, rank=r, wkind="outlier")
        codes, scales, st = O.quantize(0, w)
        q = qweight_dev(fp4w, 0, codes, scales, st)
        y = fp4w.linear(bf16_dev(x), q, bf16_dev(a), bf16_dev(b), workspace=ws)
        torch.cuda.synchronize()
        assert _counters_zero(fp4w, ws), f"counters after m={m} n={n} k={k} r={r}"
        y64 = O.linear(0, x, codes, scales, st, a, b)
        xn = np.sqrt((f64_of_bf16(x) ** 2).sum(axis=1))[:, None]
        wn = weff_norms(0, codes, scales, st, a, b)[None, :]
        check_bound(f64_of_bf16(bits_host(y)), y64, xn, wn, f"interleaved m={m} n={n} k={k} r={r}")
