"""Output guard regions: every entry point writes its outputs and nothing
around them.

Each output is the middle of a larger allocation whose 4 KB before and
after hold a canary byte pattern; the call gets the exact-shape view (the
pads keep 256-byte alignment), and afterwards both pads must hold the
canary still. Shapes are ragged in rows, k and batch, including the batch
GEMV's split-run path that first zeroes y and then adds partial sums into
it. The guarded outputs must also equal an unguarded call's.
"""
import ctypes

import numpy as np
import pytest
import torch

import bit_gemv_amd as bg
from gpu_helpers import dev_bf16, host, say
from workloads import f32_to_bf16_bits

pytestmark = pytest.mark.gpu

PAD = 4096
CANARY = 0xA5


class Guarded:
    """A tensor of `shape` and `dtype` with canary pads on both sides."""

    def __init__(self, shape, dtype):
        self.numel = int(np.prod(shape)) if len(shape) else 1
        self.nbytes = self.numel * torch.empty((), dtype=dtype).element_size()
        self.buf = torch.full((PAD + self.nbytes + PAD,), CANARY, dtype=torch.uint8, device="cuda")
        self.t = self.buf[PAD:PAD + self.nbytes].view(dtype).view(shape)

    def ptr(self):
        return ctypes.c_void_p(self.t.data_ptr())

    def check(self, what):
        torch.cuda.synchronize()
        b = self.buf.cpu().numpy()
        head, tail = b[:PAD], b[PAD + self.nbytes:]
        assert np.all(head == CANARY), f"{what}: {np.count_nonzero(head != CANARY)} bytes before the output changed"
        assert np.all(tail == CANARY), f"{what}: {np.count_nonzero(tail != CANARY)} bytes after the output changed"


def _st():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _ok(st, fn):
    assert st == 0, f"{fn}: status {st}: {bg.load_library().lq_last_error()}"


def _w(n, k, seed):
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(rng.standard_normal((n, k)) * 0.02)


def _x(m, k, seed):
    rng = np.random.default_rng(seed + 1)
    return f32_to_bf16_bits(rng.standard_normal((m, k)))


@pytest.mark.parametrize("bits,sym,group", [(4, False, 128), (4, True, 256), (8, False, 128), (8, True, "k")])
@pytest.mark.parametrize("n,k", [(37, 384), (1031, 2048 + 640)])
def test_quantize_and_dequantize(n, k, bits, sym, group):
    group = k if group == "k" else group
    if k % group:
        pytest.skip("group does not divide k")
    lib = bg.load_library()
    w = dev_bf16(_w(n, k, n + k))
    say(f"guard quantize/dequantize n={n} k={k} bits={bits} sym={sym} group={group}")
    cb = (n, k // 2 if bits == 4 else k)
    codes, scales = Guarded(cb, torch.uint8), Guarded((n, k // group), torch.float32)
    zeros = None if sym else Guarded((n, k // group), torch.float32)
    _ok(lib.quantize_groupwise(_p(w), n, k, bits, int(sym), group, None, codes.ptr(), scales.ptr(),
                               None if sym else zeros.ptr(), _st()), "quantize_groupwise")
    for g, nm in ((codes, "codes"), (scales, "scales"), (zeros, "zeros")):
        if g is not None:
            g.check(nm)
    ref = bg.quantize_groupwise(w, bits, sym, group)
    assert torch.equal(codes.t, ref.codes) and torch.equal(scales.t.view(torch.int32), ref.scales.view(torch.int32))
    out = Guarded((n, k), torch.float32)
    _ok(lib.dequantize_groupwise(codes.ptr(), scales.ptr(), None if sym else zeros.ptr(), n, k, bits, int(sym), group,
                                 out.ptr(), _st()), "dequantize_groupwise")
    out.check("dequantized")
    assert torch.equal(out.t, bg.dequantize_groupwise(ref))


@pytest.mark.parametrize("b", [1, 3, 4, 9, 16])
@pytest.mark.parametrize("n,k", [(37, 384), (1031, 2048 + 640), (4096 + 17, 11008)])
def test_weight_only_gemv(n, k, b):
    """W4A16 and W8A16 GEMV; (4096 + 17) x 11008 at batch 4..16 takes the
    shared-stage kernel's split runs (y zeroed, partial sums added)."""
    lib = bg.load_library()
    w = dev_bf16(_w(n, k, n))
    x = dev_bf16(_x(b, k, b))
    for bits, fn, ref_fn in ((4, "w4a16_gemv", bg.w4a16_gemv), (8, "w8a16_gemv", bg.w8a16_gemv)):
        pw = bg.quantize_groupwise(w, bits, False, 128)
        say(f"guard {fn} n={n} k={k} b={b}")
        y = Guarded((b, n), torch.float32)
        _ok(getattr(lib, fn)(_p(x), b, _p(pw.codes), _p(pw.scales), _p(pw.zeros), n, k, 0, 128, y.ptr(), _st()), fn)
        y.check(f"{fn} y")
        yr = ref_fn(x, pw)
        assert torch.allclose(y.t, yr, rtol=1e-5, atol=1e-6 * float(yr.abs().max()))


@pytest.mark.parametrize("m,n,k", [(5, 33, 384), (257, 300, 2048 + 128)])
def test_prefill_gemms(m, n, k):
    lib = bg.load_library()
    w = dev_bf16(_w(n, k, m))
    x = dev_bf16(_x(m, k, n))
    pw = bg.quantize_groupwise(w, 4, False, 128)
    say(f"guard w4a16_gemm / mxfp4_gemm m={m} n={n} k={k}")
    y = Guarded((m, n), torch.float32)
    _ok(lib.w4a16_gemm(_p(x), m, _p(pw.codes), _p(pw.scales), _p(pw.zeros), n, k, 0, 128, y.ptr(), _st()),
        "w4a16_gemm")
    y.check("w4a16_gemm y")
    assert torch.equal(y.t, bg.w4a16_gemm(x, pw))
    mw = bg.mxfp4_quantize(w)
    y2 = Guarded((m, n), torch.float32)
    _ok(lib.mxfp4_gemm(_p(x), m, _p(mw.codes), _p(mw.scales), n, k, y2.ptr(), _st()), "mxfp4_gemm")
    y2.check("mxfp4_gemm y")
    assert torch.equal(y2.t, bg.mxfp4_gemm(x, mw))


@pytest.mark.parametrize("b", [1, 5, 16])
@pytest.mark.parametrize("n,k", [(37, 384), (4096 + 17, 11008)])
def test_mxfp4_quantize_and_gemv(n, k, b):
    lib = bg.load_library()
    w = dev_bf16(_w(n, k, k))
    say(f"guard mxfp4 n={n} k={k} b={b}")
    codes, scales = Guarded((n, k // 2), torch.uint8), Guarded((n, k // 32), torch.uint8)
    _ok(lib.mxfp4_quantize(_p(w), n, k, codes.ptr(), scales.ptr(), _st()), "mxfp4_quantize")
    codes.check("mx codes")
    scales.check("mx scales")
    x = dev_bf16(_x(b, k, k))
    y = Guarded((b, n), torch.float32)
    _ok(lib.mxfp4_gemv(_p(x), b, codes.ptr(), scales.ptr(), n, k, y.ptr(), _st()), "mxfp4_gemv")
    y.check("mxfp4_gemv y")


def test_smoothquant_chain():
    lib = bg.load_library()
    t, n, k = 77, 300, 1024 + 128
    x = dev_bf16(_x(t, k, 3))
    w = dev_bf16(_w(n, k, 4))
    say("guard smooth_scale / quant_per_token_int8 / w8a8_gemm")
    s = Guarded((k,), torch.float32)
    _ok(lib.smooth_scale(_p(x), t, _p(w), n, k, ctypes.c_float(0.5), s.ptr(), _st()), "smooth_scale")
    s.check("smooth s")
    qx, sx = Guarded((t, k), torch.int8), Guarded((t,), torch.float32)
    _ok(lib.quant_per_token_int8(_p(x), t, k, s.ptr(), qx.ptr(), sx.ptr(), _st()), "quant_per_token_int8")
    qx.check("qx")
    sx.check("sx")
    pw = bg.quantize_groupwise(w, 8, True, k, s.t)
    acc, y = Guarded((t, n), torch.int32), Guarded((t, n), torch.float32)
    _ok(lib.w8a8_gemm(qx.ptr(), sx.ptr(), t, _p(pw.codes), _p(pw.scales), n, k, acc.ptr(), y.ptr(), _st()),
        "w8a8_gemm")
    acc.check("w8a8 acc")
    y.check("w8a8 y")


def test_gptq_and_awq():
    lib = bg.load_library()
    t, n, k = 96, 300, 1024
    x = dev_bf16(_x(t, k, 5))
    w = dev_bf16(_w(n, k, 6))
    say("guard gptq_hessian_factor / gptq_quantize(_noalloc) / act_absmean / awq_search")
    u = Guarded((k, k), torch.float32)
    ws = torch.empty(lib.gptq_workspace_bytes(t, n, k), dtype=torch.uint8, device="cuda")
    _ok(lib.gptq_hessian_factor(_p(x), t, k, ctypes.c_float(0.01), _p(ws), ws.numel(), u.ptr(), _st()),
        "gptq_hessian_factor")
    u.check("U")
    for noalloc in (False, True):
        codes, scales, zeros = (Guarded((n, k // 2), torch.uint8), Guarded((n, k // 128), torch.float32),
                                Guarded((n, k // 128), torch.float32))
        if noalloc:
            st = lib.gptq_quantize_noalloc(_p(w), n, k, u.ptr(), 4, 0, 128, codes.ptr(), scales.ptr(), zeros.ptr(),
                                           _st())
        else:
            st = lib.gptq_quantize(_p(w), n, k, u.ptr(), 4, 0, 128, _p(ws), ws.numel(), codes.ptr(), scales.ptr(),
                                   zeros.ptr(), _st())
        _ok(st, "gptq_quantize")
        for g, nm in ((codes, "codes"), (scales, "scales"), (zeros, "zeros")):
            g.check(f"gptq {nm} (noalloc={noalloc})")
    sxa = Guarded((k,), torch.float32)
    _ok(lib.act_absmean(_p(x), t, k, sxa.ptr(), _st()), "act_absmean")
    sxa.check("act_absmean")
    n_grid = 4
    wsa = torch.empty(lib.awq_workspace_bytes(t, n, k), dtype=torch.uint8, device="cuda")
    s_best, losses, best = (Guarded((k,), torch.float32), Guarded((n_grid + 1,), torch.float64),
                            Guarded((1,), torch.int32))
    codes, scales, zeros = (Guarded((n, k // 2), torch.uint8), Guarded((n, k // 128), torch.float32),
                            Guarded((n, k // 128), torch.float32))
    _ok(lib.awq_search(_p(x), t, _p(w), n, k, 0, 128, n_grid, sxa.ptr(), _p(wsa), wsa.numel(), s_best.ptr(),
                       losses.ptr(), best.ptr(), codes.ptr(), scales.ptr(), zeros.ptr(), _st()), "awq_search")
    for g, nm in ((s_best, "s_best"), (losses, "losses"), (best, "best"), (codes, "codes"), (scales, "scales"),
                  (zeros, "zeros")):
        g.check(f"awq {nm}")
