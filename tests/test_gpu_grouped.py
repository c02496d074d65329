"""GPU parity of the grouped (MoE) W4A16 linear against the binary64 oracle:
128 experts with gate/up (768, 2048) and down (2048, 768) weights, 64 tokens
routed top-8; plus empty experts, experts with more than 16 rows, a single
expert, out-of-range token indices (NaN rows), offsets outside [0, total rows]
(clamped; rows no expert covers keep their contents) and a K above 4096 (the
per-tile kernel instead of the x-in-registers one)."""
import numpy as np
import pytest
import torch

import oracle as O
from mxfp4_bit_weight_amd import workloads as W
from tests.gpu_util import DEV, Guarded, bf16_dev, bits_host, check_bound, f32_dev, f64_of_bf16, i32_dev, say, u8_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp4w():
    from mxfp4_bit_weight_amd import fp4w as F
    return F


def _experts(fmt, seed, e, n, k):
    wts = W.moe_expert_weights(seed, e, n, k)
    q = [O.quantize(fmt, wts[i]) for i in range(e)]
    return (np.stack([c for c, _, _ in q]), np.stack([s for _, s, _ in q]),
            np.array([t for _, _, t in q], np.float32))


def _case(fp4w, fmt, x, row_index, offsets, codes, scales, ts, what):
    say(f"[grouped] {what} fmt={fmt} experts={codes.shape[0]} n={codes.shape[1]} k={codes.shape[2] * 2} rows={row_index.size}")
    g = Guarded((row_index.size, codes.shape[1]), torch.bfloat16, float("nan"))
    y = fp4w.grouped_linear(bf16_dev(x), i32_dev(row_index), i32_dev(offsets), fmt, u8_dev(codes), u8_dev(scales),
                            f32_dev(ts) if fmt == 0 else None, out=g.t)
    g.check(f"grouped {what}")
    yg = f64_of_bf16(bits_host(y))
    y64 = O.grouped_linear(fmt, x, row_index, offsets, codes, scales, ts)
    xn = np.sqrt((f64_of_bf16(x) ** 2).sum(axis=1))[row_index][:, None]
    wn = np.zeros((row_index.size, codes.shape[1]))
    for e in range(codes.shape[0]):
        if offsets[e + 1] > offsets[e]:
            d = O.dequantize(fmt, codes[e], scales[e], ts[e], "f64")
            wn[offsets[e]:offsets[e + 1]] = np.sqrt((d * d).sum(axis=1))[None, :]
    check_bound(yg, y64, xn, wn, what)


@pytest.mark.parametrize("fmt", [0, 1])
def test_moe_gate_and_down(fp4w, fmt):
    cfg = W.MOE
    row_index, offsets = W.moe_routing(0)
    assert row_index.size == cfg["tokens"] * cfg["topk"]
    x = W.normal_bf16(0, W.TID_X, (cfg["tokens"], cfg["d_model"]), 1.0)
    codes, scales, ts = _experts(fmt, 0, cfg["experts"], cfg["d_ff"], cfg["d_model"])
    _case(fp4w, fmt, x, row_index, offsets, codes, scales, ts, "gate (768, 2048)")
    # down projection: input rows are the routed rows themselves (identity index)
    xd = W.normal_bf16(0, W.TID_DOWN_IN, (row_index.size, cfg["d_ff"]), 1.0)
    codes, scales, ts = _experts(fmt, 1, cfg["experts"], cfg["d_model"], cfg["d_ff"])
    _case(fp4w, fmt, xd, np.arange(row_index.size, dtype=np.int32), offsets, codes, scales, ts, "down (2048, 768)")


@pytest.mark.parametrize("fmt", [0, 1])
def test_uneven_routing(fp4w, fmt):
    # expert 0: 40 rows (three chunks of up to 16), expert 1: 0 rows, expert 2: 1 row, expert 3: 13 rows
    counts = np.array([40, 0, 1, 13])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rng = np.random.default_rng(9)
    row_index = rng.integers(0, 30, offsets[-1]).astype(np.int32)
    x = W.normal_bf16(2, W.TID_X, (30, 544), 1.0)
    codes, scales, ts = _experts(fmt, 2, 4, 70, 544)
    _case(fp4w, fmt, x, row_index, offsets, codes, scales, ts, "uneven routing")


# Each expert's rows go through runs of up to 6 weight tiles of 16 rows: fewer
# than 96 rows take runs of 1 to 5 (n = 9, 20, 40, 64: 1, 2, 3 and 4 tiles, the
# last one ragged where n is not a multiple of 16), K with and without staged
# scales (512: 16-byte scale rows; 544: not).
@pytest.mark.parametrize("n,k", [(9, 512), (20, 544), (40, 512), (64, 544)])
@pytest.mark.parametrize("fmt", [0, 1])
def test_few_tiles_per_expert(fp4w, fmt, n, k):
    offsets = np.array([0, 17, 17, 20], np.int32)
    rng = np.random.default_rng(n)
    row_index = rng.integers(0, 12, offsets[-1]).astype(np.int32)
    x = W.normal_bf16(5, W.TID_X, (12, k), 1.0)
    codes, scales, ts = _experts(fmt, 5, 3, n, k)
    _case(fp4w, fmt, x, row_index, offsets, codes, scales, ts, f"{n} rows per expert")


@pytest.mark.parametrize("fmt", [0, 1])
def test_long_k_uses_the_per_tile_kernel(fp4w, fmt):
    # K = 4160: 130 groups of 32, more than one span of the x-in-registers kernel holds
    offsets = np.array([0, 5, 5, 22], np.int32)
    rng = np.random.default_rng(12)
    row_index = rng.integers(0, 9, offsets[-1]).astype(np.int32)
    x = W.normal_bf16(4, W.TID_X, (9, 4160), 1.0)
    codes, scales, ts = _experts(fmt, 4, 3, 40, 4160)
    _case(fp4w, fmt, x, row_index, offsets, codes, scales, ts, "K 4160")


@pytest.mark.parametrize("fmt", [0, 1])
def test_offsets_are_clamped(fp4w, fmt):
    """Offsets [-3, 2, 9] over 5 rows act as [0, 2, 5]; offsets [0, 2, 3] leave
    rows 3 and 4 as they were."""
    rng = np.random.default_rng(13)
    row_index = rng.integers(0, 6, 5).astype(np.int32)
    x = W.normal_bf16(5, W.TID_X, (6, 256), 1.0)
    codes, scales, ts = _experts(fmt, 5, 2, 24, 256)
    args = (u8_dev(codes), u8_dev(scales), f32_dev(ts) if fmt == 0 else None)
    y = fp4w.grouped_linear(bf16_dev(x), i32_dev(row_index), i32_dev(np.array([-3, 2, 9], np.int32)), fmt, *args)
    torch.cuda.synchronize()
    y64 = O.grouped_linear(fmt, x, row_index, np.array([0, 2, 5], np.int32), codes, scales, ts)
    xn = np.sqrt((f64_of_bf16(x) ** 2).sum(axis=1))[row_index][:, None]
    wn = np.zeros((5, 24))
    for e, (a, b) in enumerate([(0, 2), (2, 5)]):
        d = O.dequantize(fmt, codes[e], scales[e], ts[e], "f64")
        wn[a:b] = np.sqrt((d * d).sum(axis=1))[None, :]
    check_bound(f64_of_bf16(bits_host(y)), y64, xn, wn, "clamped offsets")
    out = torch.full((5, 24), 7.0, dtype=torch.bfloat16, device=DEV)
    fp4w.grouped_linear(bf16_dev(x), i32_dev(row_index), i32_dev(np.array([0, 2, 3], np.int32)), fmt, *args, out=out)
    torch.cuda.synchronize()
    assert bool((out[3:] == 7.0).all().item())
    y64 = O.grouped_linear(fmt, x, row_index[:3], np.array([0, 2, 3], np.int32), codes, scales, ts)
    check_bound(f64_of_bf16(bits_host(out[:3])), y64, xn[:3], wn[:3], "rows 0-2 of the short offsets")


@pytest.mark.parametrize("fmt", [0, 1])
def test_bad_token_index_gives_nan_rows(fp4w, fmt):
    offsets = np.array([0, 3, 5], np.int32)
    row_index = np.array([0, 99, 1, -1, 2], np.int32)
    x = W.normal_bf16(3, W.TID_X, (4, 64), 1.0)
    codes, scales, ts = _experts(fmt, 3, 2, 16, 64)
    y = fp4w.grouped_linear(bf16_dev(x), i32_dev(row_index), i32_dev(offsets), fmt, u8_dev(codes), u8_dev(scales),
                            f32_dev(ts) if fmt == 0 else None)
    torch.cuda.synchronize()
    yh = y.float().cpu().numpy()
    assert np.isnan(yh[1]).all() and np.isnan(yh[3]).all()
    assert np.isfinite(yh[[0, 2, 4]]).all()


def test_binding_rejects_bad_shapes_before_launch(fp4w):
    """Shapes the kernels index with are checked before any launch: a narrower x,
    short offsets, scales of the other format, a short tensor-scale vector or a
    wrongly sized output raise ValueError; without ``out`` y starts as zeros."""
    e, n, k = 3, 32, 256
    codes = torch.zeros((e, n, k // 2), dtype=torch.uint8, device=DEV)
    sc_nv = torch.full((e, n, k // 16), 0x38, dtype=torch.uint8, device=DEV)
    sc_mx = torch.full((e, n, k // 32), 127, dtype=torch.uint8, device=DEV)
    ts = torch.ones(e, dtype=torch.float32, device=DEV)
    x = torch.ones((4, k), dtype=torch.bfloat16, device=DEV)
    ri = torch.zeros(6, dtype=torch.int32, device=DEV)
    off = torch.tensor([0, 2, 4, 6], dtype=torch.int32, device=DEV)
    bad = [
        dict(x=x[:, :k - 32].contiguous()),                                  # narrower x
        dict(expert_offsets=off[:3].contiguous()),                            # num_experts entries only
        dict(scales=sc_mx),                                                   # MXFP4-shaped scales with NVFP4
        dict(tensor_scales=ts[:2].contiguous()),                              # one tensor scale short
        dict(tensor_scales=None),                                             # NVFP4 without tensor scales
        dict(codes=codes.view(torch.int8)),                                   # not uint8
        dict(out=torch.empty((6, n - 1), dtype=torch.bfloat16, device=DEV)),  # short output rows
    ]
    base = dict(x=x, row_index=ri, expert_offsets=off, fmt=0, codes=codes, scales=sc_nv, tensor_scales=ts)
    for change in bad:
        args = dict(base, **change)
        with pytest.raises(ValueError):
            fp4w.grouped_linear(**args)
    with pytest.raises(ValueError):
        fp4w.grouped_linear(**dict(base, fmt=1))                              # NVFP4-shaped scales with MXFP4
    y = fp4w.grouped_linear(**dict(base, expert_offsets=torch.tensor([0, 1, 2, 3], dtype=torch.int32,
                                                                        device=DEV)))
    torch.cuda.synchronize()
    assert bool((y[3:] == 0).all().item()), "rows no expert covers must read as zero"
