"""Helpers for the GPU parity tests: host <-> device transfers of bit patterns,
the oracle-side reference values, and the floating-point acceptance bound.

Acceptance for the linear (the bound the build states for floating point): every
output satisfies |y_gpu - y64| <= 2e-3 * ||x_m||_2 * ||w_n^eff||_2, where y64 is
the binary64 oracle and w_n^eff = deq(W)[n, :] + (B A)[n, :] in binary64.
"""
import sys

import numpy as np
import torch

import oracle as O
from mxfp4_bit_weight_amd import workloads as W

REL_TOL = 2e-3
DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(DEV)


def u8_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def f32_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.float32))).to(DEV)


def i32_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def bits_host(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64_of_bf16(bits: np.ndarray) -> np.ndarray:
    return W.bf16_bits_to_f32(bits).astype(np.float64)


def qweight_host(q):
    st = np.float32(q.tensor_scale.item()) if q.tensor_scale is not None else np.float32(1.0)
    return q.codes.cpu().numpy(), q.scales.cpu().numpy(), st


def qweight_dev(fp4w, fmt, codes, scales, st):
    n, kh = codes.shape
    return fp4w.QWeight(fmt, u8_dev(codes), u8_dev(scales), f32_dev([st]) if fmt == fp4w.NVFP4 else None,
                        n, kh * 2)


def weff_norms(fmt, codes, scales, st, a=None, b=None, rows=None):
    """||deq(W)[n] + (B A)[n]||_2 in binary64 for the given rows (all if None)."""
    if rows is None:
        rows = np.arange(codes.shape[0])
    deq = O.dequantize(fmt, codes[rows], scales[rows], st, "f64")
    if a is not None:
        deq = deq + f64_of_bf16(b[rows]) @ f64_of_bf16(a)
    return np.sqrt((deq * deq).sum(axis=1))


def check_bound(y_gpu: np.ndarray, y64: np.ndarray, xnorm: np.ndarray, wnorm: np.ndarray, what: str):
    """Element-wise acceptance; xnorm/wnorm broadcast against y."""
    bound = REL_TOL * xnorm * wnorm
    err = np.abs(y_gpu - y64)
    bad = ~(err <= bound)
    if bad.any():
        i = np.argmax(np.where(bad, err / np.maximum(bound, 1e-300), 0))
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outputs outside the bound; worst "
                             f"err={err.flat[i]:.3e} bound={bound.flat[i]:.3e} gpu={y_gpu.flat[i]!r} "
                             f"ref={y64.flat[i]!r}")
    return float((err / np.maximum(bound, 1e-300)).max()) * REL_TOL


# ---- canary bytes around device outputs ------------------------------------------------
CANARY_BYTES = 256          # on each side; keeps the output 256-byte aligned
CANARY = 0xA5


class Guarded:
    """A device output of `shape` and `dtype` inside a larger byte buffer whose
    CANARY_BYTES before and after it hold CANARY; check() asserts that no kernel
    wrote outside the output.  `fill` (a float, e.g. NaN) pre-fills the output."""

    def __init__(self, shape, dtype, fill=None):
        nbytes = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.buf = torch.full((nbytes + 2 * CANARY_BYTES,), CANARY, dtype=torch.uint8, device=DEV)
        self.nbytes = nbytes
        self.t = self.buf[CANARY_BYTES:CANARY_BYTES + nbytes].view(dtype).view(shape)
        if fill is not None:
            self.t.fill_(fill)

    def check(self, what=""):
        torch.cuda.synchronize()
        head = self.buf[:CANARY_BYTES].cpu().numpy()
        tail = self.buf[CANARY_BYTES + self.nbytes:].cpu().numpy()
        assert (head == CANARY).all() and (tail == CANARY).all(), f"{what}: bytes outside the output were written"


def guarded_qweight(fp4w, fmt, n, k):
    """An empty QWeight whose codes, scales and tensor scale are Guarded; returns
    (qweight, [guards])."""
    blk = 16 if fmt == 0 else 32
    gc = Guarded((n, k // 2), torch.uint8)
    gs = Guarded((n, k // blk), torch.uint8)
    gt = Guarded((1,), torch.float32) if fmt == 0 else None
    q = fp4w.QWeight(fmt, gc.t, gs.t, gt.t if gt is not None else None, n, k)
    return q, [g for g in (gc, gs, gt) if g is not None]
