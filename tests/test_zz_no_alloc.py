"""fp4w_linear_noalloc -- the linear with its workspace in the library's own
per-device array, for callers that cannot allocate -- against fp4w_linear.

Both entry points run the same plan and kernels, and the linear's results do not
depend on scheduling (cross-workgroup sums in a fixed order), so the outputs must
be bit for bit equal.  Each case is two calls in a row on the shared array, the
second with a smaller input, so a counter or partial left over by the first
would show in the second; one case is also checked against the oracle.  A call
that needs more than the array holds is refused before any launch."""
import numpy as np
import pytest
import torch

import oracle as O
from mxfp4_bit_weight_amd import workloads as W
from tests.gpu_util import DEV, bf16_dev, bits_host, check_bound, f64_of_bf16, qweight_dev, say, weff_norms

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp4w():
    from mxfp4_bit_weight_amd import fp4w as F
    return F


def _prepare(fp4w, fmt, m, n, k, r, seed):
    w, x, a, b = W.linear_inputs(seed, n, k, m, rank=r, wkind="outlier" if fmt == 0 else "student_t")
    codes, scales, st = O.quantize(fmt, w)
    q = qweight_dev(fp4w, fmt, codes, scales, st)
    dev = (bf16_dev(x), q, bf16_dev(a) if r else None, bf16_dev(b) if r else None)
    return dev, (x, codes, scales, st, a, b)


def _pair(fp4w, fmt, m, n, k, r, seed):
    (xd, q, ad, bd), host = _prepare(fp4w, fmt, m, n, k, r, seed)
    y_ref = fp4w.linear(xd, q, ad, bd)
    y = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=DEV)
    fp4w.linear_noalloc(xd, q, ad, bd, out=y)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), f"fmt={fmt} m={m} n={n} k={k} r={r}"
    return y, host


# (first call, second smaller call): the m = 1 hand-over, the 2-16-row kernel with
# split-K partials, the GEMM with t in the array, and a switch between paths
PAIRS = [
    ((1, 18944, 3584, 16), (1, 3584, 3584, 16)),
    ((8, 3584, 18944, 16), (4, 1000, 2080, 17)),
    ((16, 3584, 18944, 64), (8, 3584, 3584, 16)),
    ((600, 520, 1280, 17), (40, 64, 256, 5)),
    ((300, 1030, 1056, 16), (1, 200, 544, 1)),
]


@pytest.mark.parametrize("first,second", PAIRS)
@pytest.mark.parametrize("fmt", [0, 1])
def test_noalloc_matches_linear_on_two_calls(fp4w, fmt, first, second):
    say(f"[noalloc] fmt={fmt} {first} then {second}")
    _pair(fp4w, fmt, *first, seed=sum(first))
    y, (x, codes, scales, st, a, b) = _pair(fp4w, fmt, *second, seed=sum(second))
    m, n = y.shape
    y64 = O.linear(fmt, x, codes, scales, st, a, b)
    xn = np.sqrt((f64_of_bf16(x) ** 2).sum(axis=1))[:, None]
    wn = weff_norms(fmt, codes, scales, st, a, b)[None, :]
    check_bound(f64_of_bf16(bits_host(y)), y64, xn, wn, f"noalloc second call m={m} n={n}")


def test_noalloc_refuses_calls_beyond_its_array(fp4w):
    """m * r * 4 bytes of t past the array's 8 MiB: refused with its own status,
    the output untouched."""
    m, n, k, r = 40000, 64, 256, 64
    assert fp4w.linear_workspace_bytes(m, n, k, r) > fp4w.NOALLOC_SCRATCH_BYTES
    (xd, q, ad, bd), _ = _prepare(fp4w, 0, m, n, k, r, 5)
    y = torch.full((m, n), 7.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(fp4w.Fp4wError) as e:
        fp4w.linear_noalloc(xd, q, ad, bd, out=y)
    assert e.value.status == -7
    torch.cuda.synchronize()
    assert bool((y == 7.0).all().item())
