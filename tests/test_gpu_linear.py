"""GPU parity of the W4A16 linear (decode-shaped kernel for m <= 16, MFMA GEMM
for m > 16) against the binary64 oracle, within |err| <= 2e-3 ||x_m|| ||w_n^eff||.

Ragged shapes (rows not a multiple of the 16-row tile, K not a multiple of the
128-wide step, odd LoRA ranks) run against the full oracle; the full-size decode
and prefill shapes run on sampled outputs the oracle computes one by one."""
import numpy as np
import pytest
import torch

import oracle as O
from mxfp4_bit_weight_amd import workloads as W
from tests.gpu_util import (Guarded, DEV, bf16_dev, bits_host, check_bound, f64_of_bf16, qweight_dev, say,
                            weff_norms)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp4w():
    from mxfp4_bit_weight_amd import fp4w as F
    return F


def _run_dev(fp4w, fmt, w, x, a, b, nan_out=False):
    codes, scales, st = O.quantize(fmt, w)
    q = qweight_dev(fp4w, fmt, codes, scales, st)
    g = Guarded((x.shape[0], q.n), torch.bfloat16, float("nan") if nan_out else None)
    y = fp4w.linear(bf16_dev(x), q, bf16_dev(a) if a is not None else None, bf16_dev(b) if b is not None else None,
                    out=g.t)
    g.check(f"linear fmt={fmt} m={x.shape[0]} n={q.n} k={q.k}")
    return y, codes, scales, st


def _run(fp4w, fmt, w, x, a, b, nan_out=False):
    y, codes, scales, st = _run_dev(fp4w, fmt, w, x, a, b, nan_out=nan_out)
    return f64_of_bf16(bits_host(y)), codes, scales, st


def _full_case(fp4w, fmt, m, n, k, r, seed=0, wkind="normal", nan_out=False):
    say(f"[linear] fmt={fmt} m={m} n={n} k={k} r={r} seed={seed}")
    w, x, a, b = W.linear_inputs(seed, n, k, m, rank=r, wkind=wkind)
    yg, codes, scales, st = _run(fp4w, fmt, w, x, a, b, nan_out=nan_out)
    y64 = O.linear(fmt, x, codes, scales, st, a, b)
    xn = np.sqrt((f64_of_bf16(x) ** 2).sum(axis=1))[:, None]
    wn = weff_norms(fmt, codes, scales, st, a, b)[None, :]
    return check_bound(yg, y64, xn, wn, f"m={m} n={n} k={k} r={r}")


@pytest.mark.parametrize("fmt", [0, 1])
def test_single_linear(fp4w, fmt):
    """W 256x512 ~ N(0, 0.02), x 1x512 ~ N(0, 1), LoRA r = 16, seed 0."""
    worst = _full_case(fp4w, fmt, 1, 256, 512, 16)
    say(f"  worst relative error {worst:.2e}")


SKINNY = [(1, 200, 544, 16), (2, 45, 96, 5), (3, 1000, 1056, 64), (4, 17, 32, 0), (5, 300, 4128, 16),
          (7, 64, 256, 1), (8, 1000, 2080, 16), (11, 33, 640, 16), (16, 257, 1024, 32)]


@pytest.mark.parametrize("m,n,k,r", SKINNY)
@pytest.mark.parametrize("fmt", [0, 1])
def test_skinny_ragged(fp4w, fmt, m, n, k, r):
    _full_case(fp4w, fmt, m, n, k, r, seed=m * 7 + r, wkind="outlier")


# The 2-16-row kernel gives each workgroup a run of 1 to 6 weight tiles of 16
# rows, about one workgroup per compute unit (256 on MI355X, fewer the LoRA's
# chunk workgroups): n of 5000, 9000, 13000 and 22000 rows take runs of 2, 3, 4
# and 6 tiles, with and without LoRA, a ragged last tile each.  Outputs are
# NaN-filled first, so an output no run writes fails the bound.
TILE_RUNS = [(8, 5000, 512, 0), (8, 9000, 512, 16), (8, 13000, 512, 16), (16, 22000, 512, 0), (3, 22000, 256, 16)]


@pytest.mark.parametrize("m,n,k,r", TILE_RUNS)
@pytest.mark.parametrize("fmt", [0, 1])
def test_skinny_tile_runs(fp4w, fmt, m, n, k, r):
    _full_case(fp4w, fmt, m, n, k, r, seed=n + r, wkind="outlier", nan_out=True)


GEMM = [(17, 300, 256, 16), (100, 520, 1056, 16), (300, 257, 544, 0), (64, 64, 64, 5), (513, 700, 2048, 64)]
# K a multiple of 128 (the GEMM that decodes W in registers): ragged rows and
# columns over several 256 x 256 tiles, n not a multiple of 4 (element stores),
# the shortest K (one weight stage), LoRA ranks not a multiple of 8
GEMM_W4 = [(257, 301, 256, 5), (600, 520, 1280, 17), (33, 1030, 512, 1), (300, 257, 768, 0), (40, 64, 256, 64)]


@pytest.mark.parametrize("m,n,k,r", GEMM)
@pytest.mark.parametrize("fmt", [0, 1])
def test_gemm_ragged(fp4w, fmt, m, n, k, r):
    _full_case(fp4w, fmt, m, n, k, r, seed=m + r, wkind="outlier")


@pytest.mark.parametrize("m,n,k,r", GEMM_W4)
@pytest.mark.parametrize("fmt", [0, 1])
def test_gemm_k256(fp4w, fmt, m, n, k, r):
    _full_case(fp4w, fmt, m, n, k, r, seed=m + 3 * r, wkind="outlier" if fmt == 0 else "student_t")


@pytest.mark.parametrize("fmt", [0, 1])
def test_gemm_more_tiles_than_cus(fp4w, fmt):
    """17 x 17 = 289 tiles of 256 x 256, more than the 256 workgroups of one per
    CU, so workgroups take several tiles: every output is written (y starts as
    NaN) and 4096 sampled outputs are within the bound."""
    m = n = 17 * 256 - 40
    k, seed = 384, 77
    say(f"[linear] many tiles fmt={fmt} m={m} n={n} k={k}")
    w, x, a, b = W.linear_inputs(seed, n, k, m, rank=16, wkind="outlier" if fmt == 0 else "student_t")
    codes, scales, st = O.quantize(fmt, w)
    q = qweight_dev(fp4w, fmt, codes, scales, st)
    y = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=DEV)
    fp4w.linear(bf16_dev(x), q, bf16_dev(a), bf16_dev(b), out=y)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all().item()), "an output was not written"
    rng = np.random.default_rng(seed)
    rows = rng.integers(0, m, 4096)
    cols = rng.integers(0, n, 4096)
    ys = f64_of_bf16(bits_host(y[torch.from_numpy(rows).to(DEV), torch.from_numpy(cols).to(DEV)]))
    y64 = O.linear_sampled(fmt, x, codes, scales, st, rows, cols, a, b)
    xn = np.sqrt((f64_of_bf16(x[rows]) ** 2).sum(axis=1))
    wn = weff_norms(fmt, codes, scales, st, a, b, rows=cols)
    check_bound(ys, y64, xn, wn, f"many tiles fmt={fmt}")


def _sampled_case(fp4w, fmt, m, n, k, samples, seed, what):
    say(f"[linear] {what} fmt={fmt} m={m} n={n} k={k} (sampled)")
    wkind = "outlier" if fmt == 0 else "student_t"
    w, x, a, b = W.linear_inputs(seed, n, k, m, rank=16, wkind=wkind)
    yd, codes, scales, st = _run_dev(fp4w, fmt, w, x, a, b, nan_out=True)   # y starts as NaN
    rng = np.random.default_rng(seed)
    rows = rng.integers(0, m, samples)
    cols = rng.integers(0, n, samples)
    ys = f64_of_bf16(bits_host(yd[torch.from_numpy(rows).to(DEV), torch.from_numpy(cols).to(DEV)]))
    assert bool(torch.isfinite(yd).all().item()), "an output was not written"
    del yd
    y64 = O.linear_sampled(fmt, x, codes, scales, st, rows, cols, a, b)
    xn = np.sqrt((f64_of_bf16(x[rows]) ** 2).sum(axis=1))
    wn = weff_norms(fmt, codes, scales, st, a, b, rows=cols)
    check_bound(ys, y64, xn, wn, what)


@pytest.mark.parametrize("name", ["gate_up", "down", "qkv_o"])
@pytest.mark.parametrize("m", [1, 8])
@pytest.mark.parametrize("fmt", [0, 1])
def test_decode_full_size(fp4w, fmt, m, name):
    n, k = W.QWEN7B_SHAPES[name]
    _sampled_case(fp4w, fmt, m, n, k, 1024, seed=21, what=f"Qwen-2.5-7B {name}")


def test_prefill_gemm_full_size(fp4w):
    """x 16384 x 3584, W (18944, 3584) NVFP4, LoRA r = 16; 4096 sampled outputs."""
    n, k = W.QWEN7B_SHAPES["gate_up"]
    _sampled_case(fp4w, 0, W.PREFILL_M, n, k, 4096, seed=31, what="prefill 8x2048")


def test_workspace_counters_return_to_zero_and_determinism(fp4w):
    say("[linear] workspace + determinism")
    n, k, m = 3584, 18944, 4                     # small n: split-K with arrival counters
    w, x, a, b = W.linear_inputs(41, n, k, m, rank=16)
    codes, scales, st = O.quantize(0, w)
    q = qweight_dev(fp4w, 0, codes, scales, st)
    nbytes = fp4w.linear_workspace_bytes(m, n, k, 16)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    xd, ad, bd = bf16_dev(x), bf16_dev(a), bf16_dev(b)
    y1 = fp4w.linear(xd, q, ad, bd, workspace=ws)
    y2 = fp4w.linear(xd, q, ad, bd, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    # the counter area (arrival counters, LoRA hand-over words) must be zero again
    counters = ws[:fp4w.WORKSPACE_COUNTER_BYTES].view(torch.int32)
    assert int(counters.abs().sum().item()) == 0


def test_workspace_reuse_across_shapes(fp4w):
    """One workspace serving calls of different shapes: counters and partials of
    one call must not disturb the next (the counters sit at fixed offsets)."""
    say("[linear] workspace reuse across shapes")
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device=DEV)
    for (m, n, k, r) in [(8, 1000, 2080, 16), (11, 33, 640, 16), (4, 3584, 4096, 16), (11, 33, 640, 16),
                         (1, 200, 544, 16), (16, 257, 1024, 32)]:
        w, x, a, b = W.linear_inputs(m * 7 + r, n, k, m, rank=r, wkind="outlier")
        codes, scales, st = O.quantize(0, w)
        q = qweight_dev(fp4w, 0, codes, scales, st)
        y = fp4w.linear(bf16_dev(x), q, bf16_dev(a), bf16_dev(b), workspace=ws)
        torch.cuda.synchronize()
        y64 = O.linear(0, x, codes, scales, st, a, b)
        xn = np.sqrt((f64_of_bf16(x) ** 2).sum(axis=1))[:, None]
        wn = weff_norms(0, codes, scales, st, a, b)[None, :]
        check_bound(f64_of_bf16(bits_host(y)), y64, xn, wn, f"reuse m={m} n={n} k={k}")
        assert int(ws[:fp4w.WORKSPACE_COUNTER_BYTES].view(torch.int32).abs().sum().item()) == 0


@pytest.mark.parametrize("fmt", [0, 1])
def test_empty_k_writes_zeros(fp4w, fmt):
    """k == 0: every output is an empty sum, so y = 0 whatever the path m picks
    (the operands are never read; non-null stand-ins satisfy the argument checks)."""
    n = 40
    stand = torch.zeros(4096, dtype=torch.uint8, device=DEV)
    p = fp4w._ptr(stand)
    ts = torch.ones(1, dtype=torch.float32, device=DEV)
    for m in (1, 2, 8, 16, 17):
        for r in (0, 16):
            say(f"empty k: fmt={fmt} m={m} r={r}")
            g = Guarded((m, n), torch.bfloat16, float("nan"))
            nb = fp4w.linear_workspace_bytes(m, n, 0, r)
            ws = torch.zeros(nb, dtype=torch.uint8, device=DEV)
            rc = fp4w._linear(fmt, p, m, 0, p, p, fp4w._ptr(ts) if fmt == 0 else None, n, p if r else None,
                              p if r else None, r, fp4w._ptr(g.t), fp4w._ptr(ws), nb, fp4w._stream(DEV))
            assert rc == 0, rc
            torch.cuda.synchronize()
            g.check(f"empty k fmt={fmt} m={m} r={r}")
            assert int((g.t.view(torch.int16) != 0).sum().item()) == 0
            assert int(ws.to(torch.int32).sum().item()) == 0


def test_empty_and_tiny(fp4w):
    w, x, a, b = W.linear_inputs(1, 32, 64, 1, rank=16)
    codes, scales, st = O.quantize(0, w)
    q = qweight_dev(fp4w, 0, codes, scales, st)
    y = fp4w.linear(bf16_dev(x)[:0], q)
    assert y.shape == (0, 32)
    _full_case(fp4w, 0, 1, 1, 32, 0)
    _full_case(fp4w, 1, 1, 1, 32, 1)
