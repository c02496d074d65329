"""CPU oracle for NVFP4 / MXFP4 weights and the W4A16 linear.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
CPU-baseline leg of the benchmark may import this module.  It wraps
``fp4_oracle.c`` (plain C, binary64) through ctypes; see that file's header for
what each function follows on the pages and which readings it takes.

Arrays are numpy: bf16 tensors are ``uint16`` bit patterns, codes and scales
``uint8``.  ``fmt`` is 0 for NVFP4 and 1 for MXFP4.
"""
import ctypes
import os

import numpy as np

NVFP4 = 0
MXFP4 = 1
BLOCK = {NVFP4: 16, MXFP4: 32}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")


def _load():
    alt = os.environ.get("FP4W_ORACLE_LIB")        # the sanitized build (tests/run_sanitized.sh)
    if alt:
        return ctypes.CDLL(alt)
    if not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(os.path.join(_HERE, "fp4_oracle.c"))):
        from . import build as _b
        _b.build()
    return ctypes.CDLL(_LIB_PATH)


_lib = _load()

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_dbl = ctypes.c_double
_flt = ctypes.c_float


def _sig(name, restype, *argtypes):
    f = getattr(_lib, name)
    f.restype = restype
    f.argtypes = list(argtypes)
    return f


_sig("orc_init", None)
_sig("orc_e2m1_decode", _dbl, _int)
_sig("orc_e4m3_decode", _dbl, _int)
_sig("orc_e8m0_decode", _dbl, _int)
_sig("orc_e2m1_rne_quot", _int, _dbl, _dbl)
_sig("orc_e4m3_rne_quot", _int, _dbl, _dbl)
_sig("orc_round_bf16", ctypes.c_uint16, _dbl)
_sig("orc_mxfp4_scale_code", _int, _dbl)
_sig("orc_merge_scale", _int, _int, _int, _flt)
_sig("orc_nvfp4_tensor_scale", _flt, _p, _i64)
_sig("orc_nvfp4_quantize", None, _p, _i64, _i64, _p, _p, _p)
_sig("orc_nvfp4_quantize_frozen", None, _p, _i64, _i64, _p, _flt, _p)
_sig("orc_nvfp4_quantize_with_tensor_scale", None, _p, _i64, _i64, _flt, _p, _p)
_sig("orc_mxfp4_quantize", None, _p, _i64, _i64, _p, _p)
_sig("orc_mxfp4_quantize_frozen", None, _p, _i64, _i64, _p, _p)
_sig("orc_dequantize_f64", None, _int, _p, _p, _flt, _i64, _i64, _p)
_sig("orc_dequantize_f32", None, _int, _p, _p, _flt, _i64, _i64, _p)
_sig("orc_dequantize_bf16", None, _int, _p, _p, _flt, _i64, _i64, _p)
_sig("orc_merge_scales", None, _int, _p, _p, _i64, _p, _p, _p, _i64)
_sig("orc_linear", None, _int, _p, _i64, _i64, _p, _p, _flt, _i64, _p, _p, _int, _p)
_sig("orc_linear_sampled", None, _int, _p, _i64, _i64, _p, _p, _flt, _i64, _p, _p, _int,
     _p, _p, _i64, _p)
_sig("orc_grouped_linear", None, _int, _p, _p, _p, _i64, _i64, _i64, _p, _p, _p, _p)
_sig("orc_num_threads", _int)
_lib.orc_init()


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check_scales(fmt, scales, n, k):
    """The C code reads (n, k / blk) scale bytes: refuse any other shape."""
    if fmt not in BLOCK:
        raise ValueError(f"unknown format {fmt}")
    if scales.shape != (n, k // BLOCK[fmt]):
        raise ValueError(f"scales must be {(n, k // BLOCK[fmt])} for format {fmt}, got {scales.shape}")


# ---- scalar codecs ---------------------------------------------------------

def e2m1_decode(code: int) -> float:
    return _lib.orc_e2m1_decode(int(code))


def e4m3_decode(code: int) -> float:
    return _lib.orc_e4m3_decode(int(code))


def e8m0_decode(code: int) -> float:
    return _lib.orc_e8m0_decode(int(code))


def e2m1_rne_quot(a: float, d: float) -> int:
    """Magnitude code of RNE_sat(a / d) on the E2M1 grid (a >= 0, d > 0)."""
    return _lib.orc_e2m1_rne_quot(float(a), float(d))


def e4m3_rne_quot(a: float, d: float) -> int:
    """Code of RNE_sat(a / d) on the non-negative E4M3 grid (a >= 0, d > 0)."""
    return _lib.orc_e4m3_rne_quot(float(a), float(d))


def round_bf16(v: float) -> int:
    return int(_lib.orc_round_bf16(float(v)))


def mxfp4_scale_code(amax: float) -> int:
    return _lib.orc_mxfp4_scale_code(float(amax))


def merge_scale(fmt: int, code: int, delta: float) -> int:
    return _lib.orc_merge_scale(int(fmt), int(code), float(delta))


def num_threads() -> int:
    return _lib.orc_num_threads()


# ---- tensor operations -----------------------------------------------------

def nvfp4_tensor_scale(w: np.ndarray) -> np.float32:
    w = _c(w, np.uint16)
    return np.float32(_lib.orc_nvfp4_tensor_scale(_ptr(w), w.size))


def quantize(fmt: int, w: np.ndarray):
    """Dynamic ("max") quantize of a (n, k) bf16 tensor.

    Returns (codes (n, k/2) u8, scales (n, k/blk) u8, tensor_scale float32);
    tensor_scale is 1.0 for MXFP4, which has none."""
    w = _c(w, np.uint16)
    n, k = w.shape
    codes = np.zeros((n, k // 2), np.uint8)
    scales = np.zeros((n, k // BLOCK[fmt]), np.uint8)
    if fmt == NVFP4:
        st = np.zeros(1, np.float32)
        _lib.orc_nvfp4_quantize(_ptr(w), n, k, _ptr(codes), _ptr(scales), _ptr(st))
        return codes, scales, np.float32(st[0])
    _lib.orc_mxfp4_quantize(_ptr(w), n, k, _ptr(codes), _ptr(scales))
    return codes, scales, np.float32(1.0)


def nvfp4_quantize_with_tensor_scale(w: np.ndarray, tensor_scale):
    """NVFP4 block scales and codes of rows of a tensor whose s_t is given."""
    w = _c(w, np.uint16)
    n, k = w.shape
    codes = np.zeros((n, k // 2), np.uint8)
    scales = np.zeros((n, k // 16), np.uint8)
    _lib.orc_nvfp4_quantize_with_tensor_scale(_ptr(w), n, k, float(tensor_scale), _ptr(codes), _ptr(scales))
    return codes, scales


def quantize_frozen(fmt: int, w: np.ndarray, scales: np.ndarray, tensor_scale=1.0):
    """Codes only, with the block scales (and NVFP4 tensor scale) given."""
    w = _c(w, np.uint16)
    scales = _c(scales, np.uint8)
    n, k = w.shape
    codes = np.zeros((n, k // 2), np.uint8)
    if fmt == NVFP4:
        _lib.orc_nvfp4_quantize_frozen(_ptr(w), n, k, _ptr(scales), float(tensor_scale), _ptr(codes))
    else:
        _lib.orc_mxfp4_quantize_frozen(_ptr(w), n, k, _ptr(scales), _ptr(codes))
    return codes


def dequantize(fmt: int, codes, scales, tensor_scale=1.0, out: str = "f64"):
    """Decoded weights (n, k): exact binary64 ("f64"), or rounded once (RNE) to
    binary32 ("f32") or to bf16 ("bf16", uint16 bit patterns)."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    n, k = codes.shape[0], codes.shape[1] * 2
    _check_scales(fmt, scales, n, k)
    if out == "f64":
        y = np.empty((n, k), np.float64)
        _lib.orc_dequantize_f64(fmt, _ptr(codes), _ptr(scales), float(tensor_scale), n, k, _ptr(y))
    elif out == "f32":
        y = np.empty((n, k), np.float32)
        _lib.orc_dequantize_f32(fmt, _ptr(codes), _ptr(scales), float(tensor_scale), n, k, _ptr(y))
    elif out == "bf16":
        y = np.empty((n, k), np.uint16)
        _lib.orc_dequantize_bf16(fmt, _ptr(codes), _ptr(scales), float(tensor_scale), n, k, _ptr(y))
    else:
        raise ValueError(out)
    return y


def merge_scales(fmt: int, scales, deltas, codes=None):
    """Scale-only merge: returns (new scales, copy of codes or None)."""
    scales = _c(scales, np.uint8)
    deltas = _c(deltas, np.float32)
    assert scales.size == deltas.size
    out = np.empty_like(scales)
    codes_out = None
    if codes is not None:
        codes = _c(codes, np.uint8)
        codes_out = np.empty_like(codes)
    _lib.orc_merge_scales(fmt, _ptr(scales), _ptr(deltas), scales.size, _ptr(out),
                          _ptr(codes), _ptr(codes_out), 0 if codes is None else codes.size)
    return out, codes_out


def linear(fmt: int, x, codes, scales, tensor_scale, lora_a=None, lora_b=None):
    """y (m, n) in binary64 = x deq(W)^T + (x A^T) B^T."""
    x = _c(np.atleast_2d(x), np.uint16)
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    m, k = x.shape
    n = codes.shape[0]
    assert codes.shape[1] * 2 == k
    _check_scales(fmt, scales, n, k)
    r = 0
    if lora_a is not None:
        lora_a = _c(lora_a, np.uint16)
        lora_b = _c(lora_b, np.uint16)
        r = lora_a.shape[0]
        assert lora_a.shape == (r, k) and lora_b.shape == (n, r)
    y = np.empty((m, n), np.float64)
    _lib.orc_linear(fmt, _ptr(x), m, k, _ptr(codes), _ptr(scales), float(tensor_scale), n,
                    _ptr(lora_a), _ptr(lora_b), r, _ptr(y))
    return y


def linear_sampled(fmt: int, x, codes, scales, tensor_scale, rows, cols, lora_a=None, lora_b=None):
    """The outputs y[rows[s], cols[s]] of ``linear`` only, in binary64."""
    x = _c(np.atleast_2d(x), np.uint16)
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    rows = _c(rows, np.int64)
    cols = _c(cols, np.int64)
    m, k = x.shape
    n = codes.shape[0]
    assert codes.shape[1] * 2 == k
    _check_scales(fmt, scales, n, k)
    assert rows.shape == cols.shape
    assert rows.size == 0 or (rows.min() >= 0 and rows.max() < m and cols.min() >= 0 and cols.max() < n)
    r = 0
    if lora_a is not None:
        lora_a = _c(lora_a, np.uint16)
        lora_b = _c(lora_b, np.uint16)
        r = lora_a.shape[0]
        assert lora_a.shape == (r, k) and lora_b.shape == (n, r)
    y = np.empty(rows.size, np.float64)
    _lib.orc_linear_sampled(fmt, _ptr(x), m, k, _ptr(codes), _ptr(scales), float(tensor_scale), n,
                            _ptr(lora_a), _ptr(lora_b), r, _ptr(rows), _ptr(cols), rows.size, _ptr(y))
    return y


def linear_backward_dx(fmt: int, dy, codes, scales, tensor_scale):
    """Input gradient through the frozen quantized base (Telegram post, "Metod":
    the base stays frozen while training back-propagates through it): dX (m, k)
    in binary64 = dY deq(W), dY bf16 (m, n), W decoded exactly, one binary64
    matrix product."""
    dy = _c(np.atleast_2d(dy), np.uint16)
    dyf = (dy.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return dyf @ dequantize(fmt, codes, scales, tensor_scale, "f64")


def lora_backward(dy, x, lora_a, lora_b):
    """Gradients of the LoRA branch y_lora = (x A^T) B^T of the linear (Telegram
    post, "Metod": an adapter trained in parallel to the frozen base), in
    binary64, from the output gradient dY (m, n) and the input x (m, k), both
    bf16, A (r, k) and B (n, r) bf16:
        t  = x A^T          (m, r)
        u  = dY B           (m, r)
        dB = dY^T t         (n, r)
        dA = u^T x          (r, k)
        dX_lora = u A       (m, k)   (added to dY deq(W) for the whole input gradient)
    Returns (t, u, dA, dB, dX_lora); each is one binary64 matrix product of
    exact inputs, in the order the chain rule gives them."""
    f = lambda a: (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    dyf, xf = f(np.atleast_2d(dy)), f(np.atleast_2d(x))
    af, bf = f(lora_a), f(lora_b)
    t = xf @ af.T
    u = dyf @ bf
    db = dyf.T @ t
    da = u.T @ xf
    dx = u @ af
    return t, u, da, db, dx


def scale_delta_grad(fmt: int, dy, x, codes, tensor_scale):
    """Scale-QLoRA delta gradient (Scale-QLoRA page: block-scale corrections in
    the decoded scale domain, rounded to the grid in every forward, the rounding
    passed straight through): g[n, b] = s_t * sum_{k in b} e2m1(q[n, k]) *
    (dY^T X)[n, k], in binary64.  e2m1(q) is the oracle's decoding of the codes
    under the unit block scale (E4M3 0x38, E8M0 127)."""
    dy = _c(np.atleast_2d(dy), np.uint16)
    x = _c(np.atleast_2d(x), np.uint16)
    codes = _c(codes, np.uint8)
    n, k = codes.shape[0], codes.shape[1] * 2
    blk = BLOCK[fmt]
    unit = np.full((n, k // blk), 0x38 if fmt == NVFP4 else 127, np.uint8)
    e2m1 = dequantize(fmt, codes, unit, 1.0, "f64")
    f = lambda a: (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    gmat = f(dy).T @ f(x)
    ts = float(np.float32(tensor_scale)) if fmt == NVFP4 else 1.0
    return ts * (e2m1 * gmat).reshape(n, k // blk, blk).sum(axis=2)


def aqn_sigma(step: int, total_steps: int, sigma_max: float = 1e-2, sigma_min: float = 5e-4) -> float:
    """Noise scale on the exponential schedule from sigma_max to sigma_min
    (Telegram post, "Metod": the noise decays from 1e-2 to 5e-4 exponentially)."""
    if total_steps <= 0 or step >= total_steps:
        return sigma_min
    if step <= 0:
        return sigma_max
    return sigma_max * (sigma_min / sigma_max) ** (step / total_steps)


def aqn_rmsnorm(x, gamma, noise, sigma: float, eps: float):
    """Noisy RMSNorm ahead of the projections (Telegram post, "Metod": noise in
    the RMS norm before the projections, multiplicative on their weights), in
    binary64: y = x / sqrt(mean(x^2) + eps) * gamma * (1 + sigma * noise); x and
    gamma bf16 bit patterns, noise fp32; the reading of where the noise enters
    (a factor on the gain) is stated with the kernel's."""
    f = lambda a: (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    xf = f(np.atleast_2d(x))
    r = 1.0 / np.sqrt((xf * xf).mean(axis=1, keepdims=True) + float(np.float32(eps)))
    gain = f(gamma)[None, :] * (1.0 + float(np.float32(sigma)) * np.asarray(noise, np.float32).astype(np.float64))[None, :]
    return xf * r * gain


def linear_aqn(fmt: int, x, gamma, noise, sigma: float, eps: float, codes, scales, tensor_scale,
               lora_a=None, lora_b=None):
    """The projection of the noisy RMSNorm's output (Telegram post, "Metod": the
    noise enters the RMS norm that precedes the projections), in binary64 with
    no rounding between the two: x~ = aqn_rmsnorm(x, gamma, noise, sigma, eps),
    y = x~ deq(W)^T + (x~ A^T) B^T, W decoded exactly, LoRA A (r, k) and B (n, r)
    bf16 bit patterns or None."""
    xt = aqn_rmsnorm(x, gamma, noise, sigma, eps)
    w = dequantize(fmt, codes, scales, tensor_scale, "f64")
    y = xt @ w.T
    if lora_a is not None:
        f = lambda a: (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        y = y + (xt @ f(lora_a).T) @ f(lora_b).T
    return y


def linear_w4a4(x_codes, x_scales, codes, scales):
    """W4A4 MXFP4 (QATFactory page, section on the strategies NVFP4 and MXFP4
    need: weights and activations both 4-bit): y (m, n) in binary64 =
    deq(x) deq(W)^T, each operand decoded exactly (E2M1 code times its block's
    E8M0 scale), then one binary64 matrix product."""
    xd = dequantize(MXFP4, x_codes, x_scales, 1.0, "f64")
    wd = dequantize(MXFP4, codes, scales, 1.0, "f64")
    return xd @ wd.T


def linear_w4a4_sampled(x_codes, x_scales, codes, scales, rows, cols):
    """The outputs y[rows[s], cols[s]] of ``linear_w4a4`` only: each a binary64
    dot product of one decoded row of x and one decoded row of W."""
    x_codes, x_scales = _c(x_codes, np.uint8), _c(x_scales, np.uint8)
    codes, scales = _c(codes, np.uint8), _c(scales, np.uint8)
    rows, cols = np.asarray(rows, np.int64), np.asarray(cols, np.int64)
    xd = dequantize(MXFP4, x_codes[rows], x_scales[rows], 1.0, "f64")
    wd = dequantize(MXFP4, codes[cols], scales[cols], 1.0, "f64")
    return np.einsum("sk,sk->s", xd, wd)


def grouped_linear(fmt: int, x, row_index, offsets, codes, scales, tensor_scales):
    """MoE grouped linear: codes (E, n, k/2), scales (E, n, k/blk), tensor_scales (E,);
    rows sorted by expert with offsets (E+1,); returns y (R, n) in binary64."""
    x = _c(x, np.uint16)
    row_index = _c(row_index, np.int32)
    offsets = _c(offsets, np.int32)
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    ts = _c(tensor_scales, np.float32)
    e, n, kh = codes.shape
    k = kh * 2
    assert x.shape[1] == k and offsets.size == e + 1
    if scales.shape != (e, n, k // BLOCK[fmt]) or ts.size < e:
        raise ValueError("scales must be (experts, n, k / blk) with one tensor scale per expert")
    assert row_index.size == 0 or (row_index.min() >= 0 and row_index.max() < x.shape[0])
    total = int(offsets[-1])
    y = np.zeros((total, n), np.float64)
    _lib.orc_grouped_linear(fmt, _ptr(x), _ptr(row_index), _ptr(offsets), e, n, k,
                            _ptr(codes), _ptr(scales), _ptr(ts), _ptr(y))
    return y
