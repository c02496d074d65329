"""Thin Python binding of ``libfp4w.so`` (C ABI in ``include/fp4w.h``).

Argument marshalling only: every step runs in the library's gfx950 kernels.
PyTorch supplies device memory and the current HIP stream.  The functions carry
the C entry points' names without the ``fp4w_`` prefix.  Importing this module
fails loudly if the library has not been built (``__graft_entry__.build()`` or
``python mxfp4_bit_weight_amd/build.py``).
"""
import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

NVFP4 = 0
MXFP4 = 1
BLOCK = {NVFP4: 16, MXFP4: 32}
FROZEN_SCALES = 0x1
OUT_FP32 = 0x2
MAX_LORA_RANK = 64
# the workspace's first bytes: arrival counters and LoRA hand-over words, zero between calls
WORKSPACE_COUNTER_BYTES = 28800

_HERE = os.path.dirname(os.path.abspath(__file__))
# FP4W_LIB: another build of the same library (the host-sanitized one of tests/run_sanitized.sh)
LIB_PATH = os.environ.get("FP4W_LIB") or os.path.join(_HERE, "libfp4w.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build the HIP library first "
                      "(python mxfp4_bit_weight_amd/build.py)")
_lib = ctypes.CDLL(LIB_PATH)

_p, _i64, _int, _u32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint32, ctypes.c_size_t


def _sig(name, restype, *args):
    f = getattr(_lib, name)
    f.restype = restype
    f.argtypes = list(args)
    return f


_quantize = _sig("fp4w_quantize", _int, _int, _p, _i64, _i64, _p, _p, _p, _u32, _p)
_dequantize = _sig("fp4w_dequantize", _int, _int, _p, _p, _p, _i64, _i64, _p, _u32, _p)
_fake_quant = _sig("fp4w_fake_quant", _int, _int, _p, _i64, _i64, _p, _p, _p, _u32, _p)
_ws_bytes = _sig("fp4w_linear_workspace_bytes", _sz, _i64, _i64, _i64, _int)
_linear = _sig("fp4w_linear", _int, _int, _p, _i64, _i64, _p, _p, _p, _i64, _p, _p, _int, _p, _p, _sz, _p)
_linear_noalloc = _sig("fp4w_linear_noalloc", _int, _int, _p, _i64, _i64, _p, _p, _p, _i64, _p, _p, _int, _p, _p)
_w4a4 = _sig("fp4w_linear_w4a4", _int, _int, _p, _p, _i64, _i64, _p, _p, _i64, _p, _p)
_bwd_dx = _sig("fp4w_linear_backward_dx", _int, _int, _p, _i64, _i64, _p, _p, _p, _i64, _p, _p, _int, _p, _p)
_lora_bwd_ws = _sig("fp4w_lora_backward_workspace_bytes", _sz, _i64, _i64, _i64, _int)
_lora_bwd = _sig("fp4w_lora_backward", _int, _p, _i64, _i64, _p, _i64, _p, _p, _int, _p, _p, _p, _p, _sz, _p)
_delta_grad = _sig("fp4w_scale_delta_grad", _int, _int, _p, _p, _i64, _i64, _i64, _p, _p, _p, _p)
_aqn = _sig("fp4w_aqn_rmsnorm", _int, _p, _i64, _i64, _p, _p, ctypes.c_float, ctypes.c_float, _p, _p)
_aqn_sigma = _sig("fp4w_aqn_sigma", ctypes.c_double, _i64, _i64, ctypes.c_double, ctypes.c_double)
_linear_aqn_ws = _sig("fp4w_linear_aqn_workspace_bytes", _sz, _i64, _i64, _i64, _int)
_linear_aqn = _sig("fp4w_linear_aqn", _int, _int, _p, _i64, _i64, _p, _p, ctypes.c_float, ctypes.c_float, _p, _p, _p,
                   _i64, _p, _p, _int, _p, _p, _sz, _p)
_grouped = _sig("fp4w_grouped_linear", _int, _int, _p, _i64, _p, _p, _i64, _i64, _i64, _i64, _p, _p, _p, _p, _p)
_merge = _sig("fp4w_merge_scales", _int, _int, _p, _p, _i64, _p, _p, _p, _i64, _p)
_status = _sig("fp4w_status_string", ctypes.c_char_p, _int)
_version = _sig("fp4w_version", _int)
_debug_lora_wait = _sig("fp4w_debug_lora_wait", _i64, _i64)

EXPORTED = ["fp4w_quantize", "fp4w_dequantize", "fp4w_linear_workspace_bytes", "fp4w_linear",
            "fp4w_grouped_linear", "fp4w_merge_scales", "fp4w_status_string", "fp4w_version",
            "fp4w_debug_lora_wait", "fp4w_fake_quant", "fp4w_linear_w4a4", "fp4w_linear_backward_dx",
            "fp4w_scale_delta_grad", "fp4w_aqn_rmsnorm", "fp4w_aqn_sigma", "fp4w_linear_noalloc",
            "fp4w_lora_backward", "fp4w_lora_backward_workspace_bytes", "fp4w_linear_aqn",
            "fp4w_linear_aqn_workspace_bytes"]


class Fp4wError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {_status(status).decode()} (status {status})")
        self.status = status


def _check(status: int, what: str):
    if status != 0:
        raise Fp4wError(status, what)


def status_string(status: int) -> str:
    return _status(int(status)).decode()


def version() -> int:
    return _version()


def debug_lora_wait(ticks: int = -1) -> int:
    """Test hook: bound (100 MHz ticks) on the m = 1 decode kernel's wait for a
    published LoRA product before it forms the product itself; < 0 only queries.
    Returns the previous bound."""
    return int(_debug_lora_wait(int(ticks)))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, dtype, name):
    if t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor on the GPU")



def _out(out: Optional[torch.Tensor], shape, dtype, device, name="out") -> torch.Tensor:
    """`out` checked to be a contiguous GPU tensor of exactly `shape` and `dtype`
    (a smaller buffer would be written past its end), or a new one."""
    if out is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _need(out, dtype, name)
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(out.shape)}")
    return out

@dataclass
class QWeight:
    """A block-scaled 4-bit weight W (n, k): codes (n, k/2) uint8, scales
    (n, k/blk) uint8, and for NVFP4 a one-element fp32 tensor scale."""
    fmt: int
    codes: torch.Tensor
    scales: torch.Tensor
    tensor_scale: Optional[torch.Tensor]
    n: int
    k: int


def empty_qweight(fmt: int, n: int, k: int, device) -> QWeight:
    dev = torch.device(device)
    return QWeight(fmt, torch.empty((n, k // 2), dtype=torch.uint8, device=dev),
                   torch.empty((n, k // BLOCK[fmt]), dtype=torch.uint8, device=dev),
                   torch.empty(1, dtype=torch.float32, device=dev) if fmt == NVFP4 else None, n, k)


def _check_frozen(frozen: "QWeight", fmt: int, n: int, k: int, device) -> None:
    """Frozen scales (and NVFP4 tensor scale) must match W's shape: the kernels read them whole."""
    _out(frozen.scales, (n, k // BLOCK[fmt]), torch.uint8, device, "frozen.scales")
    if fmt == NVFP4:
        _out(frozen.tensor_scale, (1,), torch.float32, device, "frozen.tensor_scale")


def quantize(w: torch.Tensor, fmt: int = NVFP4, out: Optional[QWeight] = None,
             frozen: Optional[QWeight] = None) -> QWeight:
    """fp4w_quantize.  ``frozen``: reuse its scales (and tensor scale) and compute codes only."""
    _need(w, torch.bfloat16, "w")
    n, k = w.shape
    q = out if out is not None else empty_qweight(fmt, n, k, w.device)
    if out is not None:
        _out(out.codes, (n, k // 2), torch.uint8, w.device, "out.codes")
        if frozen is None:
            _out(out.scales, (n, k // BLOCK[fmt]), torch.uint8, w.device, "out.scales")
            if fmt == NVFP4:
                _out(out.tensor_scale, (1,), torch.float32, w.device, "out.tensor_scale")
    flags = 0
    if frozen is not None:
        flags = FROZEN_SCALES
        _check_frozen(frozen, fmt, n, k, w.device)
        q.scales, q.tensor_scale = frozen.scales, frozen.tensor_scale
    _check(_quantize(fmt, _ptr(w), n, k, _ptr(q.codes), _ptr(q.scales), _ptr(q.tensor_scale), flags,
                     _stream(w.device)), "fp4w_quantize")
    return q


def fake_quant(w: torch.Tensor, fmt: int = NVFP4, frozen: Optional[QWeight] = None,
               out: Optional[torch.Tensor] = None):
    """fp4w_fake_quant: dequantize(quantize(w)) in one pass, as bf16 (n, k).
    Returns (w_fq, scales, tensor_scale); ``frozen`` supplies the scales (and
    NVFP4 tensor scale) instead of computing them."""
    _need(w, torch.bfloat16, "w")
    n, k = w.shape
    y = _out(out, (n, k), torch.bfloat16, w.device)
    flags = 0
    if frozen is not None:
        flags = FROZEN_SCALES
        _check_frozen(frozen, fmt, n, k, w.device)
        scales, ts = frozen.scales, frozen.tensor_scale
    else:
        scales = torch.empty((n, k // BLOCK[fmt]), dtype=torch.uint8, device=w.device)
        ts = torch.empty(1, dtype=torch.float32, device=w.device) if fmt == NVFP4 else None
    _check(_fake_quant(fmt, _ptr(w), n, k, _ptr(y), _ptr(scales), _ptr(ts), flags, _stream(w.device)),
           "fp4w_fake_quant")
    return y, scales, ts


class FakeQuantSTE(torch.autograd.Function):
    """Training forward through fp4w_fake_quant; backward: the plain
    straight-through estimator (the gradient passes unchanged)."""

    @staticmethod
    def forward(ctx, w, fmt=NVFP4):
        y, _, _ = fake_quant(w.detach(), fmt)
        return y

    @staticmethod
    def backward(ctx, grad):
        return grad, None


def dequantize(q: QWeight, dtype=torch.bfloat16, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp4w_dequantize: the exact decoded values rounded once to bf16 or fp32."""
    if dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("dtype must be bfloat16 or float32")
    y = _out(out, (q.n, q.k), dtype, q.codes.device)
    _check(_dequantize(q.fmt, _ptr(q.codes), _ptr(q.scales), _ptr(q.tensor_scale), q.n, q.k, _ptr(y),
                       OUT_FP32 if dtype == torch.float32 else 0, _stream(q.codes.device)), "fp4w_dequantize")
    return y


def linear_workspace_bytes(m: int, n: int, k: int, r: int) -> int:
    return int(_ws_bytes(m, n, k, r))


_workspaces = {}


def workspace_for(device: torch.device, nbytes: int) -> torch.Tensor:
    """A zero-filled workspace per (device, current stream), grown on demand.  The
    library returns its counters to zero after every call, so it is reused as is."""
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 1 << 16), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def linear(x: torch.Tensor, q: QWeight, lora_a: Optional[torch.Tensor] = None,
           lora_b: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp4w_linear: y = x deq(W)^T + (x A^T) B^T, bf16 in and out, fp32 accumulation."""
    _need(x, torch.bfloat16, "x")
    m, k = x.shape
    if k != q.k:
        raise ValueError(f"x has k={k}, the weight k={q.k}")
    r = 0
    if lora_a is not None or lora_b is not None:
        _need(lora_a, torch.bfloat16, "lora_a")
        _need(lora_b, torch.bfloat16, "lora_b")
        r = lora_a.shape[0]
        if lora_a.shape != (r, k) or lora_b.shape != (q.n, r):
            raise ValueError("lora_a must be (r, k) and lora_b (n, r)")
    y = _out(out, (m, q.n), torch.bfloat16, x.device)
    nbytes = linear_workspace_bytes(m, q.n, k, r)
    ws = workspace if workspace is not None else workspace_for(x.device, nbytes)
    _check(_linear(q.fmt, _ptr(x), m, k, _ptr(q.codes), _ptr(q.scales), _ptr(q.tensor_scale), q.n,
                   _ptr(lora_a), _ptr(lora_b), r, _ptr(y), _ptr(ws), ws.numel(), _stream(x.device)),
           "fp4w_linear")
    return y


NOALLOC_SCRATCH_BYTES = 8 << 20


def linear_noalloc(x: torch.Tensor, q: QWeight, lora_a: Optional[torch.Tensor] = None,
                   lora_b: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp4w_linear_noalloc: fp4w_linear with the library's own per-device scratch
    array as its workspace; with ``out`` given nothing is allocated."""
    _need(x, torch.bfloat16, "x")
    m, k = x.shape
    if k != q.k:
        raise ValueError(f"x has k={k}, the weight k={q.k}")
    r = 0
    if lora_a is not None or lora_b is not None:
        _need(lora_a, torch.bfloat16, "lora_a")
        _need(lora_b, torch.bfloat16, "lora_b")
        r = lora_a.shape[0]
        if lora_a.shape != (r, k) or lora_b.shape != (q.n, r):
            raise ValueError("lora_a must be (r, k) and lora_b (n, r)")
    y = _out(out, (m, q.n), torch.bfloat16, x.device)
    _check(_linear_noalloc(q.fmt, _ptr(x), m, k, _ptr(q.codes), _ptr(q.scales), _ptr(q.tensor_scale), q.n,
                           _ptr(lora_a), _ptr(lora_b), r, _ptr(y), _stream(x.device)), "fp4w_linear_noalloc")
    return y


def linear_w4a4(xq: QWeight, q: QWeight, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp4w_linear_w4a4: y = deq(x) deq(W)^T for x (m, k) and W (n, k) both
    MXFP4 (``xq`` as ``quantize(x, MXFP4)`` returns it), bf16 out."""
    if xq.fmt != MXFP4 or q.fmt != MXFP4:
        raise ValueError("linear_w4a4 takes MXFP4 activations and weights")
    if xq.k != q.k:
        raise ValueError(f"x has k={xq.k}, the weight k={q.k}")
    y = _out(out, (xq.n, q.n), torch.bfloat16, q.codes.device)
    _check(_w4a4(MXFP4, _ptr(xq.codes), _ptr(xq.scales), xq.n, xq.k, _ptr(q.codes), _ptr(q.scales), q.n,
                 _ptr(y), _stream(y.device)), "fp4w_linear_w4a4")
    return y


def linear_a4(x: torch.Tensor, q: QWeight, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The W4A4 forward from bf16 activations: x quantized to MXFP4 (fp4w_quantize),
    then fp4w_linear_w4a4."""
    return linear_w4a4(quantize(x, MXFP4), q, out)


def linear_backward_dx(dy: torch.Tensor, q: QWeight, out: Optional[torch.Tensor] = None,
                       lora_u: Optional[torch.Tensor] = None, lora_a: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp4w_linear_backward_dx: dx = dy deq(W) (+ u A with the adapter's u = dy B
    from ``lora_backward`` and its A), bf16 in and out, fp32 accumulation."""
    _need(dy, torch.bfloat16, "dy")
    m, n = dy.shape
    if n != q.n:
        raise ValueError(f"dy has n={n}, the weight n={q.n}")
    r = 0
    if lora_u is not None or lora_a is not None:
        _need(lora_u, torch.float32, "lora_u")
        _need(lora_a, torch.bfloat16, "lora_a")
        r = lora_a.shape[0]
        if lora_a.shape != (r, q.k) or lora_u.shape != (m, r):
            raise ValueError("lora_a must be (r, k) and lora_u (m, r)")
    dx = _out(out, (m, q.k), torch.bfloat16, dy.device)
    _check(_bwd_dx(q.fmt, _ptr(dy), m, n, _ptr(q.codes), _ptr(q.scales), _ptr(q.tensor_scale), q.k, _ptr(lora_u),
                   _ptr(lora_a), r, _ptr(dx), _stream(dy.device)), "fp4w_linear_backward_dx")
    return dx


def lora_backward_workspace_bytes(m: int, n: int, k: int, r: int) -> int:
    return int(_lora_bwd_ws(m, n, k, r))


def lora_backward(dy: torch.Tensor, x: torch.Tensor, lora_a: torch.Tensor, lora_b: torch.Tensor,
                  workspace: Optional[torch.Tensor] = None, out=None):
    """fp4w_lora_backward: (u, grad_a, grad_b) for the adapter y_lora = (x A^T) B^T,
    u = dy B (m, r), dA = u^T x (r, k), dB = dy^T (x A^T) (n, r), all fp32."""
    _need(dy, torch.bfloat16, "dy")
    _need(x, torch.bfloat16, "x")
    _need(lora_a, torch.bfloat16, "lora_a")
    _need(lora_b, torch.bfloat16, "lora_b")
    m, n = dy.shape
    r, k = lora_a.shape
    if x.shape != (m, k) or lora_b.shape != (n, r):
        raise ValueError("dy (m, n), x (m, k), lora_a (r, k) and lora_b (n, r) must agree")
    dev = dy.device
    if out is not None:                                  # (u, grad_a, grad_b), fp32, contiguous
        u = _out(out[0], (m, r), torch.float32, dev, "u")
        ga = _out(out[1], (r, k), torch.float32, dev, "grad_a")
        gb = _out(out[2], (n, r), torch.float32, dev, "grad_b")
    else:
        u = torch.empty((m, r), dtype=torch.float32, device=dev)
        ga = torch.empty((r, k), dtype=torch.float32, device=dev)
        gb = torch.empty((n, r), dtype=torch.float32, device=dev)
    nbytes = lora_backward_workspace_bytes(m, n, k, r)
    if nbytes == 0:
        raise ValueError("invalid lora_backward shape")
    ws = workspace if workspace is not None else torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _check(_lora_bwd(_ptr(dy), m, n, _ptr(x), k, _ptr(lora_a), _ptr(lora_b), r, _ptr(u), _ptr(ga), _ptr(gb),
                     _ptr(ws), ws.numel(), _stream(dev)), "fp4w_lora_backward")
    return u, ga, gb


def scale_delta_grad(dy: torch.Tensor, x: torch.Tensor, q: QWeight, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp4w_scale_delta_grad: the gradient of the Scale-QLoRA block-scale deltas,
    fp32 (n, k / blk), from the output gradient dy (m, n) and the input x (m, k)."""
    _need(dy, torch.bfloat16, "dy")
    _need(x, torch.bfloat16, "x")
    m, n = dy.shape
    if n != q.n or x.shape != (m, q.k):
        raise ValueError("dy must be (m, n) and x (m, k) for the weight (n, k)")
    g = _out(out, (q.n, q.k // BLOCK[q.fmt]), torch.float32, dy.device)
    _check(_delta_grad(q.fmt, _ptr(dy), _ptr(x), m, n, q.k, _ptr(q.codes), _ptr(q.tensor_scale), _ptr(g),
                       _stream(dy.device)), "fp4w_scale_delta_grad")
    return g


def aqn_sigma(step: int, total_steps: int, sigma_max: float = 1e-2, sigma_min: float = 5e-4) -> float:
    """fp4w_aqn_sigma: the exponentially decaying noise scale."""
    return float(_aqn_sigma(step, total_steps, sigma_max, sigma_min))


def linear_aqn_workspace_bytes(m: int, n: int, k: int, r: int = 0) -> int:
    return int(_linear_aqn_ws(m, n, k, r))


def linear_aqn(x: torch.Tensor, gamma: torch.Tensor, noise: torch.Tensor, sigma: float, q: QWeight,
               lora_a: Optional[torch.Tensor] = None, lora_b: Optional[torch.Tensor] = None, eps: float = 1e-6,
               out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp4w_linear_aqn: the linear of the noisy RMSNorm of x (the norm fused into
    the decode kernels where each workgroup covers the whole K, m <= 16)."""
    _need(x, torch.bfloat16, "x")
    _need(gamma, torch.bfloat16, "gamma")
    _need(noise, torch.float32, "noise")
    m, k = x.shape
    if k != q.k:
        raise ValueError(f"x has k={k}, the weight k={q.k}")
    if gamma.shape != (k,) or noise.shape != (k,):
        raise ValueError("gamma and noise must be (k,)")
    r = 0
    if lora_a is not None or lora_b is not None:
        _need(lora_a, torch.bfloat16, "lora_a")
        _need(lora_b, torch.bfloat16, "lora_b")
        r = lora_a.shape[0]
        if lora_a.shape != (r, k) or lora_b.shape != (q.n, r):
            raise ValueError("lora_a must be (r, k) and lora_b (n, r)")
    y = _out(out, (m, q.n), torch.bfloat16, x.device)
    nbytes = linear_aqn_workspace_bytes(m, q.n, k, r)
    ws = workspace if workspace is not None else workspace_for(x.device, nbytes)
    _check(_linear_aqn(q.fmt, _ptr(x), m, k, _ptr(gamma), _ptr(noise), float(sigma), float(eps), _ptr(q.codes),
                       _ptr(q.scales), _ptr(q.tensor_scale), q.n, _ptr(lora_a), _ptr(lora_b), r, _ptr(y), _ptr(ws),
                       ws.numel(), _stream(x.device)), "fp4w_linear_aqn")
    return y


def aqn_rmsnorm(x: torch.Tensor, gamma: torch.Tensor, noise: torch.Tensor, sigma: float, eps: float = 1e-6,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp4w_aqn_rmsnorm: RMSNorm with the per-channel gain gamma * (1 + sigma * noise)."""
    _need(x, torch.bfloat16, "x")
    _need(gamma, torch.bfloat16, "gamma")
    _need(noise, torch.float32, "noise")
    m, k = x.shape
    if gamma.numel() != k or noise.numel() != k:
        raise ValueError("gamma and noise must have k elements")
    y = _out(out, (m, k), torch.bfloat16, x.device)
    _check(_aqn(_ptr(x), m, k, _ptr(gamma), _ptr(noise), float(sigma), float(eps), _ptr(y), _stream(x.device)),
           "fp4w_aqn_rmsnorm")
    return y


def grouped_linear(x: torch.Tensor, row_index: torch.Tensor, expert_offsets: torch.Tensor, fmt: int,
                   codes: torch.Tensor, scales: torch.Tensor, tensor_scales: Optional[torch.Tensor],
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp4w_grouped_linear over experts: codes (E, n, k/2), scales (E, n, k/blk).

    Every shape the kernels index with is checked before the launch (a narrower
    x, short offsets or scales of the other format would be read past their
    ends).  Without ``out``, y is zero-filled first, so rows no expert covers
    read as zero rather than as stale memory."""
    if fmt not in BLOCK:
        raise ValueError(f"unknown format {fmt}")
    _need(x, torch.bfloat16, "x")
    _need(row_index, torch.int32, "row_index")
    _need(expert_offsets, torch.int32, "expert_offsets")
    _need(codes, torch.uint8, "codes")
    _need(scales, torch.uint8, "scales")
    if codes.dim() != 3:
        raise ValueError("codes must be (num_experts, n, k/2)")
    e, n, kh = codes.shape
    k = kh * 2
    if x.dim() != 2 or x.shape[1] != k:
        raise ValueError(f"x must be (num_tokens, {k}), got {tuple(x.shape)}")
    if row_index.dim() != 1:
        raise ValueError("row_index must be one-dimensional")
    if expert_offsets.shape != (e + 1,):
        raise ValueError(f"expert_offsets must hold num_experts + 1 = {e + 1} entries, "
                         f"got {tuple(expert_offsets.shape)}")
    if tuple(scales.shape) != (e, n, k // BLOCK[fmt]):
        raise ValueError(f"scales must be {(e, n, k // BLOCK[fmt])} for this format, got {tuple(scales.shape)}")
    if fmt == NVFP4:
        if tensor_scales is None:
            raise ValueError("NVFP4 needs one tensor scale per expert")
        _need(tensor_scales, torch.float32, "tensor_scales")
        if tensor_scales.numel() != e:
            raise ValueError(f"tensor_scales must hold {e} entries, got {tensor_scales.numel()}")
    total = row_index.numel()
    y = torch.zeros((total, n), dtype=torch.bfloat16, device=x.device) if out is None else \
        _out(out, (total, n), torch.bfloat16, x.device)
    _check(_grouped(fmt, _ptr(x), x.shape[0], _ptr(row_index), _ptr(expert_offsets), e, total, n, k,
                    _ptr(codes), _ptr(scales), _ptr(tensor_scales) if fmt == NVFP4 else None, _ptr(y),
                    _stream(x.device)), "fp4w_grouped_linear")
    return y


def merge_scales(q: QWeight, deltas: torch.Tensor, in_place: bool = False,
                 scales_out: Optional[torch.Tensor] = None) -> QWeight:
    """fp4w_merge_scales: new scales on the format's grid.  ``in_place``: q's
    scales are overwritten; ``scales_out``: written there, codes shared;
    otherwise a new QWeight whose codes are copied byte for byte.  The tensor
    scale is shared in every case."""
    _need(deltas, torch.float32, "deltas")
    if deltas.numel() != q.scales.numel():
        raise ValueError("one delta per block scale")
    if in_place or scales_out is not None:
        dst = q.scales if in_place else scales_out
        _need(dst, torch.uint8, "scales_out")
        if dst.numel() != q.scales.numel():
            raise ValueError("scales_out must hold one byte per block")
        _check(_merge(q.fmt, _ptr(q.scales), _ptr(deltas), q.scales.numel(), _ptr(dst), None, None, 0,
                      _stream(q.codes.device)), "fp4w_merge_scales")
        return q if in_place else QWeight(q.fmt, q.codes, dst, q.tensor_scale, q.n, q.k)
    new = QWeight(q.fmt, torch.empty_like(q.codes), torch.empty_like(q.scales), q.tensor_scale, q.n, q.k)
    _check(_merge(q.fmt, _ptr(q.scales), _ptr(deltas), q.scales.numel(), _ptr(new.scales), _ptr(q.codes),
                  _ptr(new.codes), q.codes.numel(), _stream(q.codes.device)), "fp4w_merge_scales")
    return new
