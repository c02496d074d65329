"""The library's kernels captured in a HIP graph: every replay, with the program's
own eager work and synchronizations between replays, must give the eager
result bit for bit (split-K arrival counters and the LoRA partials included)."""
import numpy as np
import pytest
import torch

import oracle as O
from mxfp4_bit_weight_amd import workloads as W
from tests.gpu_util import DEV, bf16_dev, qweight_dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp4w():
    from mxfp4_bit_weight_amd import fp4w as F
    return F


def _case(fp4w, fmt, m, n, k, r, seed):
    w, x, a, b = W.linear_inputs(seed, n, k, m, rank=r, wkind="outlier")
    codes, scales, st = O.quantize(fmt, w)
    q = qweight_dev(fp4w, fmt, codes, scales, st)
    return q, bf16_dev(x), bf16_dev(a), bf16_dev(b)


@pytest.mark.parametrize("fmt", [0, 1])
def test_linear_graph_replays(fp4w, fmt):
    say(f"[graph] linear fmt={fmt}")
    cases = [(1, 3584, 18944, 16), (8, 1000, 2080, 16), (1, 256, 512, 16), (40, 300, 1056, 16)]
    ws = torch.zeros(max(fp4w.linear_workspace_bytes(m, n, k, r) for m, n, k, r in cases), dtype=torch.uint8,
                     device=DEV)
    prepared = [_case(fp4w, fmt, m, n, k, r, seed=i + 10) for i, (m, n, k, r) in enumerate(cases)]
    outs = [torch.empty((x.shape[0], q.n), dtype=torch.bfloat16, device=DEV) for q, x, a, b in prepared]

    def run_all():
        for (q, x, a, b), y in zip(prepared, outs):
            fp4w.linear(x, q, a, b, out=y, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_all()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_all()
    rng = np.random.default_rng(0)
    for rep in range(5):
        # new activations, then the eager reference on the same workspace
        for (q, x, a, b) in prepared:
            x.copy_(torch.from_numpy(rng.standard_normal(tuple(x.shape)).astype(np.float32)).to(DEV).to(torch.bfloat16))
        ref = [fp4w.linear(x, q, a, b, workspace=ws) for (q, x, a, b) in prepared]
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (y, yr) in enumerate(zip(outs, ref)):
            assert torch.equal(y.view(torch.int16), yr.view(torch.int16)), f"replay {rep} case {cases[i]}"
    assert int(ws[:fp4w.WORKSPACE_COUNTER_BYTES].view(torch.int32).abs().sum().item()) == 0


@pytest.mark.parametrize("fmt", [0, 1])
def test_quantize_graph_replays(fp4w, fmt):
    say(f"[graph] quantize fmt={fmt}")
    w = bf16_dev(W.outlier_weights(3, 0, (512, 2048)))
    q = fp4w.empty_qweight(fmt, 512, 2048, DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fp4w.quantize(w, fmt, out=q)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fp4w.quantize(w, fmt, out=q)
    rng = np.random.default_rng(1)
    for rep in range(4):
        w.copy_(torch.from_numpy((rng.standard_normal((512, 2048)) * 0.02 * (rep + 1)).astype(np.float32))
                .to(DEV).to(torch.bfloat16))
        ref = fp4w.quantize(w, fmt)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(q.codes, ref.codes) and torch.equal(q.scales, ref.scales)
        if fmt == 0:
            assert torch.equal(q.tensor_scale, ref.tensor_scale)
