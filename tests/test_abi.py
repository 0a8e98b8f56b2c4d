"""CPU checks of the C-ABI library: it loads, exports every entry point the
header declares, and rejects bad arguments before any HIP call.

No compute call runs here. Calls with valid arguments are made only when no
GPU is visible, where they must report LQ_ERR_NO_DEVICE without launching.
"""
import ctypes
import os
import re

import pytest
import torch

import bit_gemv_amd as bg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libquant.h")

P = ctypes.c_void_p
A16 = P(1 << 20)          # a 16-byte-aligned fake address (never dereferenced)
B16 = P(2 << 20)
C16 = P(3 << 20)
D16 = P(4 << 20)
MIS = P((5 << 20) + 2)    # misaligned


@pytest.fixture(scope="module")
def lib():
    return bg.load_library()


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:lq_status|const char \*|int64_t|int)\s*\*?\s*(\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for ep in bg.ENTRY_POINTS:
        assert ep in names
    assert {"lq_status_string", "lq_last_error", "lq_abi_version"} <= set(names)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_exported_dynamic_symbols_are_exactly_c_names():
    out = os.popen(f"nm -D --defined-only {bg.LIB_PATH}").read()
    syms = set(re.findall(r" T (\w+)$", out, re.M))
    for name in _declared_functions():
        assert name in syms, name


def test_status_strings(lib):
    assert lib.lq_abi_version() == 1
    assert lib.lq_status_string(0) == b"ok"
    assert lib.lq_status_string(1) == b"invalid argument"
    assert lib.lq_status_string(2) == b"unsupported"
    assert lib.lq_status_string(4) == b"no device"


def _q(lib, w=A16, n=4, k=256, bits=4, sym=0, group=128, cs=None, codes=B16, scales=C16, zeros=D16):
    return lib.quantize_groupwise(w, n, k, bits, sym, group, cs, codes, scales, zeros, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(bits=5), 1),
    (dict(bits=2), 1),
    (dict(k=300, group=128), 1),              # k not a multiple of group
    (dict(group=0), 1),
    (dict(n=-1), 1),
    (dict(k=0), 1),
    (dict(group=64, k=256), 2),               # not a multiple of 128: unsupported
    (dict(w=None), 1),
    (dict(w=MIS), 1),
    (dict(codes=MIS), 1),
    (dict(sym=1), 1),                          # zeros given for symmetric
    (dict(zeros=None), 1),                     # zeros missing for asymmetric
    (dict(cs=P((6 << 20) + 4)), 1),            # col_scale not 16-byte aligned
    (dict(codes=P((1 << 20) + 64)), 1),        # codes overlap w
    (dict(scales=D16, zeros=D16), 1),          # two outputs overlap
])
def test_quantize_rejects(lib, kwargs, status):
    assert _q(lib, **kwargs) == status
    assert lib.lq_last_error() != b""


def test_empty_work_is_ok(lib):
    assert _q(lib, w=None, n=0, codes=None, scales=None, zeros=None) == 0
    assert lib.w4a16_gemv(None, 0, None, None, None, 8, 256, 1, 128, None, None) == 0
    assert lib.w8a16_gemv(None, 0, None, None, None, 8, 256, 1, 128, None, None) == 0
    assert lib.w4a16_gemm(None, 5, None, None, None, 0, 256, 1, 128, None, None) == 0
    assert lib.quant_per_token_int8(None, 0, 256, None, None, None, None) == 0
    assert lib.w8a8_gemm(None, None, 0, None, None, 4, 256, None, None, None) == 0


@pytest.mark.parametrize("args,status", [
    ((A16, 17, B16, C16, None, 8, 256, 1, 128, D16), 2),   # batch > 16
    ((A16, -1, B16, C16, None, 8, 256, 1, 128, D16), 1),
    ((A16, 1, B16, C16, D16, 8, 256, 1, 128, P(5 << 20)), 1),  # zeros for symmetric
    ((A16, 1, B16, C16, None, 8, 256, 0, 128, D16), 1),       # zeros missing
    ((MIS, 1, B16, C16, None, 8, 256, 1, 128, D16), 1),
    ((A16, 1, B16, C16, None, 8, 200, 1, 100, D16), 2),       # group not a multiple of 128
    ((A16, 1, B16, C16, None, 8, 256, 1, 128, A16), 1),       # y aliases x
])
@pytest.mark.parametrize("fn", ["w4a16_gemv", "w8a16_gemv"])
def test_gemv_rejects(lib, fn, args, status):
    assert getattr(lib, fn)(*args, None) == status


def test_w8a16_gemv_checks_overlap_with_one_byte_codes(lib):
    """INT8 codes take n * k bytes: an output starting half-way through them
    overlaps (it would not for INT4's n * k / 2)."""
    n, k = 8, 256
    codes = 2 << 20
    y = P(codes + n * k // 2 + 16)
    x, scales = P(1 << 20), P(3 << 20)
    assert lib.w8a16_gemv(x, 1, P(codes), scales, None, n, k, 1, 128, y, None) == 1
    assert b"overlap" in lib.lq_last_error()
    if torch.cuda.device_count() == 0:
        assert lib.w4a16_gemv(x, 1, P(codes), scales, None, n, k, 1, 128, y, None) == 4


def test_gemm_rejects_k_beyond_32bit_tile_offsets(lib):
    """A 128-row bf16 activation tile of k = 2^24 spans exactly 2^32 bytes,
    past the kernel's 32-bit buffer offsets: refused, largest k below works
    its way to the device check."""
    k = 1 << 24
    x, codes, scales, y = P(1 << 40), P(2 << 40), P(3 << 40), P(4 << 40)
    assert lib.w4a16_gemm(x, 1, codes, scales, None, 8, k, 1, 128, y, None) == 2
    if torch.cuda.device_count() == 0:
        assert lib.w4a16_gemm(x, 1, codes, scales, None, 8, k - 128, 1, 128, y, None) == 4


def test_smoothquant_entry_points_reject(lib):
    assert lib.smooth_scale(A16, 0, B16, 8, 256, ctypes.c_float(0.5), C16, None) == 1
    assert lib.smooth_scale(A16, 8, B16, 8, 256, ctypes.c_float(1.5), C16, None) == 1
    assert lib.smooth_scale(A16, 8, B16, 8, 200, ctypes.c_float(0.5), C16, None) == 2
    assert lib.quant_per_token_int8(A16, 4, 256, P((7 << 20) + 8), B16, C16, None) == 1
    assert lib.w8a8_gemm(A16, B16, 4, C16, D16, 4, 131072 + 128, None, P(9 << 20), None) == 2
    # k = 131072 with every code -128 would reach 2^31: rejected before any launch
    assert lib.w8a8_gemm(A16, B16, 4, C16, D16, 4, 131072, None, P(9 << 20), None) == 2
    assert b"130944" in lib.lq_last_error()
    assert lib.w8a8_gemm(A16, B16, 4, C16, D16, 4, 256, P(9 << 20), P(9 << 20), None) == 1


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a GPU is visible: valid calls would launch")
def test_valid_call_without_device_reports_no_device(lib):
    assert _q(lib) == 4
    assert b"no HIP device" in lib.lq_last_error()


def test_act_absmean_rejects(lib):
    assert lib.act_absmean(None, 4, 256, C16, None) == 1
    assert lib.act_absmean(A16, 0, 256, C16, None) == 1
    assert lib.act_absmean(A16, 4, 256, MIS, None) == 1
    assert lib.act_absmean(A16, 4, 256, A16, None) == 1  # sx overlaps x


def test_awq_workspace_bytes(lib):
    assert lib.awq_workspace_bytes(0, 8, 256) == -1
    assert lib.awq_workspace_bytes(16, 8, -1) == -1
    # the reference product fp32 [t][n]; per grid point of a batch of 11:
    # X / s bf16 [t][k], s fp32 [k], codes [n][k/2], scales and zeros fp32
    # [n][k/128]; one fp64 loss partial per GEMM workgroup and point; each
    # piece 256-byte aligned
    per_point = 8192 + 1024 + 1024 + 2 * 256
    assert lib.awq_workspace_bytes(16, 8, 256) == 512 + 11 * per_point + 256


def _awq(lib, x=A16, t=16, w=B16, n=8, k=256, sym=0, group=128, n_grid=20, sx=P(6 << 20), ws=P(7 << 20),
         ws_bytes=1 << 20, s_best=P(8 << 20), losses=P(9 << 20), best=P(10 << 20), codes=P(11 << 20),
         scales=P(12 << 20), zeros=P(13 << 20)):
    return lib.awq_search(x, t, w, n, k, sym, group, n_grid, sx, ws, ws_bytes, s_best, losses, best, codes,
                          scales, zeros, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(t=0), 1),
    (dict(n=0), 1),
    (dict(n_grid=0), 1),
    (dict(n_grid=2000), 1),
    (dict(k=300), 1),                          # k not a multiple of group
    (dict(group=64), 2),
    (dict(k=1 << 24, group=128), 2),           # past the products' 32-bit tile offsets
    (dict(x=MIS), 1),
    (dict(sx=None), 1),
    (dict(ws=None), 1),
    (dict(ws=P((7 << 20) + 16)), 1),           # workspace not 256-byte aligned
    (dict(ws_bytes=1000), 1),                  # workspace too small
    (dict(sym=1), 1),                          # zeros given for symmetric
    (dict(zeros=None), 1),                     # zeros missing for asymmetric
    (dict(ws=P(1 << 20)), 1),                  # workspace overlaps x
    (dict(codes=P(8 << 20)), 1),               # codes overlap s_best
])
def test_awq_search_rejects(lib, kwargs, status):
    assert _awq(lib, **kwargs) == status
    assert lib.lq_last_error() != b""


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a GPU is visible: valid calls would launch")
def test_awq_search_valid_call_reports_no_device(lib):
    assert _awq(lib) == 4


def test_mxfp4_entry_points_reject(lib):
    assert lib.mxfp4_quantize(A16, 4, 100, B16, C16, None) == 1      # k not a multiple of 32
    assert lib.mxfp4_quantize(A16, 4, 96, B16, C16, None) == 2       # a multiple of 32, not of 128
    assert lib.mxfp4_quantize(MIS, 4, 256, B16, C16, None) == 1
    assert lib.mxfp4_quantize(A16, 4, 256, B16, P((2 << 20) + 64), None) == 1  # scales overlap codes
    assert lib.mxfp4_quantize(None, 0, 256, None, None, None) == 0
    assert lib.mxfp4_gemv(A16, 17, B16, C16, 8, 256, D16, None) == 2
    assert lib.mxfp4_gemv(A16, 1, B16, C16, 8, 200, D16, None) == 1
    assert lib.mxfp4_gemv(A16, 1, B16, MIS, 8, 256, D16, None) == 1
    assert lib.mxfp4_gemv(A16, 1, B16, C16, 8, 256, A16, None) == 1  # y aliases x
    assert lib.mxfp4_gemv(A16, 0, B16, C16, 8, 256, D16, None) == 0


def test_gptq_entry_points_reject(lib):
    ws, ws_bytes, u = P(7 << 20), 1 << 30, P(9 << 20)
    assert lib.gptq_workspace_bytes(0, 0, 256) == 0
    assert lib.gptq_workspace_bytes(-1, 4, 256) == -1
    f = lambda **kw: lib.gptq_hessian_factor(kw.get("x", A16), kw.get("t", 32), kw.get("k", 256),
                                             ctypes.c_float(kw.get("pd", 0.01)), kw.get("ws", ws),
                                             kw.get("wsb", ws_bytes), kw.get("u", u), None)
    assert f(t=0) == 1
    assert f(pd=0.0) == 1
    assert f(pd=2.0) == 1
    assert f(k=200) == 2
    assert f(x=MIS) == 1
    assert f(wsb=100) == 1
    assert f(u=P(1 << 20)) == 1                  # u overlaps x
    q = lambda **kw: lib.gptq_quantize(kw.get("w", A16), kw.get("n", 8), kw.get("k", 256), kw.get("u", u),
                                       kw.get("bits", 4), kw.get("sym", 0), kw.get("group", 128), kw.get("ws", ws),
                                       kw.get("wsb", ws_bytes), kw.get("codes", B16), kw.get("scales", C16),
                                       kw.get("zeros", D16), None)
    assert q(bits=3) == 1
    assert q(group=64) == 2
    assert q(sym=1) == 1                         # zeros given for symmetric
    assert q(wsb=10) == 1
    assert q(codes=P(9 << 20)) == 1              # codes overlap u
    assert q(n=0, w=None, codes=None) == 0
    if torch.cuda.device_count() == 0:
        assert f() == 4 and q() == 4


def test_read_probe_rejects(lib):
    lib.lq_hbm_read_probe.argtypes = [P, ctypes.c_int64, P, P]
    assert lib.lq_read_probe_sink_words() == 1024
    assert lib.lq_hbm_read_probe(A16, 0, B16, None) == 0          # empty: no-op
    assert lib.lq_hbm_read_probe(A16, 24, B16, None) == 1         # not a multiple of 16
    assert lib.lq_hbm_read_probe(MIS, 1024, B16, None) == 1       # misaligned buffer
    assert lib.lq_hbm_read_probe(A16, 1024, None, None) == 1      # no sink
    assert lib.lq_hbm_read_probe(A16, 1 << 20, P((1 << 20) + 64), None) == 1  # sink inside the buffer


def test_mxfp4_gemm_rejects(lib):
    assert lib.mxfp4_gemm(A16, 0, B16, C16, 8, 256, D16, None) == 0          # m = 0: no-op
    assert lib.mxfp4_gemm(A16, 4, B16, C16, 8, 100, D16, None) == 1          # k not a multiple of 32
    assert lib.mxfp4_gemm(A16, 4, B16, C16, 8, 160, D16, None) == 2          # multiple of 32, not of 128
    assert lib.mxfp4_gemm(A16, 4, B16, C16, 8, 1 << 24, D16, None) == 2      # k too large
    assert lib.mxfp4_gemm(MIS, 4, B16, C16, 8, 256, D16, None) == 1          # misaligned x
    assert lib.mxfp4_gemm(A16, 4, B16, C16, 8, 256, MIS, None) == 1          # misaligned y
    assert lib.mxfp4_gemm(A16, 4, B16, C16, 8, 256, P((1 << 20) + 256), None) == 1  # y overlaps x
