"""The C-ABI library loads and exports every symbol include/fp4w.h declares, and
host-side validation rejects bad arguments before any launch (no GPU needed:
every call here returns from validation)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4w.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp4w_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from mxfp4_bit_weight_amd import fp4w
    return fp4w


def test_header_declares_the_five_calls():
    names = _declared()
    for n in ["fp4w_quantize", "fp4w_dequantize", "fp4w_linear", "fp4w_grouped_linear", "fp4w_merge_scales"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(lib.LIB_PATH)
    for name in _declared():
        assert hasattr(raw, name), name
    assert set(_declared()) == set(lib.EXPORTED)


def test_status_strings(lib):
    for code in range(-7, 1):
        assert lib.status_string(code) and lib.status_string(code) != "unknown status"
    assert lib.status_string(-99) == "unknown status"
    assert lib.version() >= 1


def test_workspace_bytes(lib):
    a = lib.linear_workspace_bytes(1, 18944, 3584, 16)
    b = lib.linear_workspace_bytes(8, 3584, 18944, 16)
    c = lib.linear_workspace_bytes(16384, 18944, 3584, 16)
    assert a > 0 and b > 0 and c >= 16384 * 16 * 4
    assert lib.linear_workspace_bytes(1, 10, 64, 65) == 0          # rank above the maximum
    assert lib.linear_workspace_bytes(-1, 10, 64, 0) == 0


def test_workspace_bytes_for_empty_k(lib):
    # k == 0 has no products (y is zeros): every m plans the counter area alone,
    # also where the decode planners would split an empty K
    for m in (1, 2, 4, 8, 16, 17, 4096):
        for r in (0, 16):
            assert lib.linear_workspace_bytes(m, 64, 0, r) == lib.WORKSPACE_COUNTER_BYTES, (m, r)
            assert lib.linear_aqn_workspace_bytes(m, 64, 0, r) >= lib.WORKSPACE_COUNTER_BYTES, (m, r)


def test_workspace_covers_the_counter_area(lib):
    # arrival counters and the LoRA hand-over words sit in the first 28800 bytes
    assert lib.WORKSPACE_COUNTER_BYTES == 28800
    assert lib.linear_workspace_bytes(1, 16, 32, 0) == lib.WORKSPACE_COUNTER_BYTES


def test_lora_wait_hook(lib):
    prev = lib.debug_lora_wait()
    assert prev == 100000                                       # 1 ms of the 100 MHz clock
    assert lib.debug_lora_wait(0) == prev
    assert lib.debug_lora_wait() == 0
    assert lib.debug_lora_wait(prev) == 0
    assert lib.debug_lora_wait() == prev


def _fake(addr):
    return ctypes.c_void_p(addr)


def test_validation_errors_without_launch(lib):
    q = lib._quantize
    A = 0x10000                  # aligned fake addresses; validation fails before use
    assert q(7, _fake(A), 4, 32, _fake(A), _fake(A), _fake(A), 0, None) == -4      # format
    assert q(0, _fake(A), 4, 32, _fake(A), _fake(A), _fake(A), 0x10, None) == -4   # flag
    assert q(0, _fake(A), 4, 48, _fake(A), _fake(A), _fake(A), 0, None) == -2      # k % 32
    assert q(0, _fake(A), -1, 32, _fake(A), _fake(A), _fake(A), 0, None) == -1     # negative
    assert q(0, None, 4, 32, _fake(A), _fake(A), _fake(A), 0, None) == -1          # null w
    assert q(0, _fake(A), 4, 32, _fake(A), _fake(A), None, 0, None) == -1          # NVFP4 needs s_t
    assert q(0, _fake(A + 8), 4, 32, _fake(A), _fake(A), _fake(A), 0, None) == -3  # alignment
    assert q(0, _fake(A), 0, 32, None, None, None, 0, None) == 0                   # empty: no-op
    d = lib._dequantize
    assert d(0, _fake(A), _fake(A), None, 4, 32, _fake(A), 0, None) == -1
    assert d(1, _fake(A), _fake(A), None, 4, 32, _fake(A + 4), 0, None) == -3
    assert d(1, _fake(A), _fake(A), None, 4, 32, _fake(A), 0x1, None) == -4
    lin = lib._linear
    ws = lib.linear_workspace_bytes(2, 16, 64, 16)
    args = dict(x=_fake(A), m=2, k=64, codes=_fake(A), scales=_fake(A), ts=_fake(A), n=16,
                a=_fake(A), b=_fake(A), r=16, y=_fake(A), ws=_fake(A), wsb=ws)

    def call(**kw):
        v = dict(args, **kw)
        return lin(0, v["x"], v["m"], v["k"], v["codes"], v["scales"], v["ts"], v["n"], v["a"], v["b"], v["r"],
                   v["y"], v["ws"], v["wsb"], None)
    assert call(r=65) == -2
    assert call(k=48) == -2
    assert call(b=None) == -1
    assert call(wsb=ws - 1) == -6
    assert call(ws=None) == -6
    assert call(ws=_fake(A + 16)) == -3
    assert call(x=_fake(A + 2)) == -3
    assert call(m=0) == 0
    g = lib._grouped
    assert g(0, _fake(A), 8, None, _fake(A), 4, 8, 16, 64, _fake(A), _fake(A), _fake(A), _fake(A), None) == -1
    assert g(0, _fake(A), 8, _fake(A), _fake(A), 4, 8, 16, 60, _fake(A), _fake(A), _fake(A), _fake(A), None) == -2
    assert g(0, _fake(A), 8, _fake(A), _fake(A), 0, 8, 16, 64, _fake(A), _fake(A), _fake(A), _fake(A), None) == 0
    mg = lib._merge
    assert mg(3, _fake(A), _fake(A), 4, _fake(A), None, None, 0, None) == -4
    assert mg(0, None, _fake(A), 4, _fake(A), None, None, 0, None) == -1
    assert mg(0, _fake(A), _fake(A), 4, _fake(A), _fake(A + 1), _fake(A + 64), 16, None) == -3
    assert mg(0, _fake(A), _fake(A), 0, _fake(A), None, None, 0, None) == 0


def test_w4a4_validation_without_launch(lib):
    f = lib._w4a4
    A = 0x10000
    assert f(0, _fake(A), _fake(A), 4, 128, _fake(A), _fake(A), 4, _fake(A), None) == -4      # NVFP4
    assert f(1, _fake(A), _fake(A), -1, 128, _fake(A), _fake(A), 4, _fake(A), None) == -1    # negative
    assert f(1, _fake(A), _fake(A), 4, 96, _fake(A), _fake(A), 4, _fake(A), None) == -2      # k % 128
    assert f(1, _fake(A), _fake(A), 4, 0, _fake(A), _fake(A), 4, _fake(A), None) == -2       # k = 0
    assert f(1, _fake(A), _fake(A), 70000, 128, _fake(A), _fake(A), 70000, _fake(A), None) == -2  # y >= 4 GiB
    assert f(1, None, _fake(A), 4, 128, _fake(A), _fake(A), 4, _fake(A), None) == -1         # null
    assert f(1, _fake(A + 8), _fake(A), 4, 128, _fake(A), _fake(A), 4, _fake(A), None) == -3  # codes
    assert f(1, _fake(A), _fake(A + 2), 4, 128, _fake(A), _fake(A), 4, _fake(A), None) == -3  # scales
    assert f(1, _fake(A), _fake(A), 4, 128, _fake(A), _fake(A), 4, _fake(A + 1), None) == -3  # y
    assert f(1, None, None, 0, 128, None, None, 4, None, None) == 0                          # empty


def test_backward_delta_aqn_validation_without_launch(lib):
    A = 0x10000
    f = lib._bwd_dx
    assert f(7, _fake(A), 4, 8, _fake(A), _fake(A), _fake(A), 32, None, None, 0, _fake(A), None) == -4     # format
    assert f(0, _fake(A), -1, 8, _fake(A), _fake(A), _fake(A), 32, None, None, 0, _fake(A), None) == -1    # negative
    assert f(0, _fake(A), 4, 12, _fake(A), _fake(A), _fake(A), 32, None, None, 0, _fake(A), None) == -2    # n % 8
    assert f(0, _fake(A), 4, 8, _fake(A), _fake(A), _fake(A), 48, None, None, 0, _fake(A), None) == -2    # k % 32
    assert f(0, _fake(A), 4, 8, _fake(A), _fake(A), None, 32, None, None, 0, _fake(A), None) == -1        # NVFP4 tensor scale
    assert f(1, _fake(A + 8), 4, 8, _fake(A), _fake(A), None, 32, None, None, 0, _fake(A), None) == -3    # dy alignment
    assert f(1, _fake(A), 4, 8, _fake(A), _fake(A), None, 32, None, None, 0, _fake(A + 4), None) == -3    # dx alignment
    assert f(1, None, 0, 8, None, None, None, 32, None, None, 0, None, None) == 0                          # m = 0
    # the LoRA term: both operands or neither, rank <= 64, alignment
    assert f(0, _fake(A), 4, 8, _fake(A), _fake(A), _fake(A), 32, _fake(A), None, 16, _fake(A), None) == -1
    assert f(0, _fake(A), 4, 8, _fake(A), _fake(A), _fake(A), 32, _fake(A), _fake(A), 65, _fake(A), None) == -2
    assert f(0, _fake(A), 4, 8, _fake(A), _fake(A), _fake(A), 32, _fake(A + 2), _fake(A), 16, _fake(A), None) == -3
    assert f(0, _fake(A), 4, 8, _fake(A), _fake(A), _fake(A), 32, _fake(A), _fake(A + 1), 16, _fake(A), None) == -3
    g = lib._delta_grad
    assert g(7, _fake(A), _fake(A), 4, 8, 32, _fake(A), _fake(A), _fake(A), None) == -4
    assert g(0, _fake(A), _fake(A), 4, 12, 32, _fake(A), _fake(A), _fake(A), None) == -2   # n % 8
    assert g(0, _fake(A), _fake(A), 4, 8, 40, _fake(A), _fake(A), _fake(A), None) == -2    # k % 32
    assert g(1, None, _fake(A), 4, 8, 32, _fake(A), None, _fake(A), None) == -1            # dy null, m > 0
    assert g(1, _fake(A), _fake(A), 4, 8, 32, _fake(A), None, _fake(A + 2), None) == -3    # grad alignment
    assert g(1, None, None, 4, 0, 32, None, None, None, None) == 0                          # n = 0
    a = lib._aqn
    assert a(_fake(A), 4, 12, _fake(A), _fake(A), 0.01, 1e-6, _fake(A), None) == -2       # k % 8
    assert a(_fake(A), -1, 16, _fake(A), _fake(A), 0.01, 1e-6, _fake(A), None) == -1
    assert a(_fake(A), 4, 16, _fake(A), None, 0.01, 1e-6, _fake(A), None) == -1            # noise null
    assert a(_fake(A), 4, 16, _fake(A), _fake(A + 4), 0.01, 1e-6, _fake(A), None) == -3    # noise alignment
    assert a(None, 0, 16, None, None, 0.01, 1e-6, None, None) == 0                          # m = 0


def test_noalloc_validation_without_launch(lib):
    """fp4w_linear_noalloc checks what fp4w_linear checks, and refuses a call whose
    workspace would exceed its device array before touching the device."""
    f = lib._linear_noalloc
    A = 0x10000
    assert lib.NOALLOC_SCRATCH_BYTES == 8 << 20
    assert f(7, _fake(A), 2, 64, _fake(A), _fake(A), _fake(A), 16, None, None, 0, _fake(A), None) == -4
    assert f(0, _fake(A), 2, 48, _fake(A), _fake(A), _fake(A), 16, None, None, 0, _fake(A), None) == -2
    assert f(0, _fake(A), 2, 64, _fake(A), _fake(A), None, 16, None, None, 0, _fake(A), None) == -1
    assert f(0, _fake(A + 2), 2, 64, _fake(A), _fake(A), _fake(A), 16, None, None, 0, _fake(A), None) == -3
    assert f(0, _fake(A), 2, 64, _fake(A), _fake(A), _fake(A), 16, _fake(A), None, 16, _fake(A), None) == -1
    assert f(0, _fake(A), 0, 64, None, None, None, 16, None, None, 0, None, None) == 0
    m, n, k, r = 40000, 64, 256, 64
    assert lib.linear_workspace_bytes(m, n, k, r) > lib.NOALLOC_SCRATCH_BYTES
    assert f(0, _fake(A), m, k, _fake(A), _fake(A), _fake(A), n, _fake(A), _fake(A), r, _fake(A), None) == -7
    assert "no-allocation" in lib.status_string(-7)


def test_lora_backward_validation_without_launch(lib):
    f = lib._lora_bwd
    A = 0x10000
    ws = lib.lora_backward_workspace_bytes(64, 48, 96, 16)
    assert ws > 0 and lib.lora_backward_workspace_bytes(64, 48, 96, 0) == 0 and lib.lora_backward_workspace_bytes(4, 8, 32, 65) == 0

    def call(**kw):
        v = dict(dy=_fake(A), m=64, n=48, x=_fake(A), k=96, a=_fake(A), b=_fake(A), r=16, u=_fake(A), ga=_fake(A),
                 gb=_fake(A), ws=_fake(A), wsb=ws)
        v.update(kw)
        return f(v["dy"], v["m"], v["n"], v["x"], v["k"], v["a"], v["b"], v["r"], v["u"], v["ga"], v["gb"], v["ws"],
                 v["wsb"], None)
    assert call(m=-1) == -1
    assert call(r=0) == -2 and call(r=65) == -2
    assert call(k=80) == -2 and call(n=44) == -2
    assert call(dy=None) == -1 and call(a=None) == -1 and call(b=None) == -1
    assert call(x=_fake(A + 8)) == -3 and call(a=_fake(A + 2)) == -3 and call(b=_fake(A + 1)) == -3
    assert call(gb=_fake(A + 2)) == -3
    assert call(wsb=ws - 1) == -6 and call(ws=None) == -6
    assert call(ws=_fake(A + 16)) == -3


def test_linear_aqn_validation_without_launch(lib):
    """fp4w_linear_aqn checks what fp4w_linear checks, then gamma, noise and the
    larger workspace, before any launch."""
    f = lib._linear_aqn
    A = 0x10000
    m, n, k = 2, 16, 64
    ws = lib.linear_aqn_workspace_bytes(m, n, k, 0)
    assert ws >= lib.linear_workspace_bytes(m, n, k, 0) + m * k * 2
    assert lib.linear_aqn_workspace_bytes(1, 10, 64, 65) == 0 and lib.linear_aqn_workspace_bytes(-1, 10, 64, 0) == 0

    def call(**kw):
        v = dict(fmt=0, x=_fake(A), m=m, k=k, g=_fake(A), nz=_fake(A), codes=_fake(A), sc=_fake(A), ts=_fake(A), n=n,
                 a=None, b=None, r=0, y=_fake(A), ws=_fake(A), wsb=ws)
        v.update(kw)
        return f(v["fmt"], v["x"], v["m"], v["k"], v["g"], v["nz"], 1e-2, 1e-6, v["codes"], v["sc"], v["ts"], v["n"],
                 v["a"], v["b"], v["r"], v["y"], v["ws"], v["wsb"], None)
    assert call(fmt=7) == -4 and call(m=-1) == -1 and call(k=48) == -2
    assert call(g=None) == -1 and call(nz=None) == -1
    assert call(g=_fake(A + 2)) == -3 and call(nz=_fake(A + 4)) == -3
    assert call(wsb=ws - 1) == -6 and call(ws=None) == -6 and call(ws=_fake(A + 16)) == -3
    assert call(a=_fake(A), r=16) == -1
    assert call(m=0, x=None, y=None, g=None, nz=None) == 0
