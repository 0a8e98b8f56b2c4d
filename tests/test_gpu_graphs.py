"""HIP graph capture and replay of the entry points that the benchmark times
from graphs. Each call is captured once into a torch CUDA graph (the binding
launches on torch's current stream, which is the capture stream), then the
graph is replayed three times; before every replay the program's own eager
work overwrites the outputs and the device is synchronized, and every replay
must reproduce the outputs of the eager call. The multi-kernel calls are
among them: the split-run batch GEMVs (an output fill kernel, then partial
sums added with atomics) and the smoothing factors (a fill kernel, column
maxima, a finishing kernel). No call clears memory with a memset node.
"""
import pytest
import torch

import bit_gemv_amd as bg
from gpu_helpers import say

pytestmark = pytest.mark.gpu


def _rand_bf16(shape, seed, scale=1.0):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return (torch.randn(shape, generator=g, device="cuda") * scale).to(torch.bfloat16)


def _poison(t: torch.Tensor):
    if t.dtype.is_floating_point:
        t.fill_(float("nan"))
    else:
        t.fill_(90)


def _check_graph(what, fn, outs, rel=0.0):
    """rel = 0: every replay bit-identical to the eager call; else relative
    L2 distance at most rel (float sums whose order varies between calls)."""
    say(f"graph {what}")
    fn()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for rep in range(3):
        for o in outs:
            _poison(o)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, ref)):
            if rel == 0.0:
                assert torch.equal(o, r), f"{what}: replay {rep}, output {i} differs from the eager call"
            else:
                assert bool(torch.isfinite(o).all()), f"{what}: replay {rep}, output {i} not finite"
                err = ((o.double() - r.double()).norm() / r.double().norm()).item()
                assert err <= rel, f"{what}: replay {rep}, output {i}: rel L2 {err:.2e} > {rel}"
    del g


def _packed(n, k, bits, symmetric, group, seed):
    w = _rand_bf16((n, k), seed, 0.02)
    return bg.quantize_groupwise(w, bits, symmetric, group)


@pytest.mark.parametrize("bits,symmetric,group", [(4, False, 128), (4, True, 256), (8, False, 128), (8, True, -1)])
def test_quantize_graph(bits, symmetric, group):
    n, k = 384, 4352
    group = k if group == -1 else group
    w = _rand_bf16((n, k), 1, 0.02)
    cs = torch.rand(k, device="cuda") + 0.5 if group == k else None
    pw = bg.quantize_groupwise(w, bits, symmetric, group, cs)
    outs = [pw.codes, pw.scales] + ([] if pw.zeros is None else [pw.zeros])
    _check_graph(f"quantize_groupwise bits={bits} sym={symmetric} G={group}",
                 lambda: bg.quantize_groupwise(w, bits, symmetric, group, cs, out=pw), outs)


def test_dequantize_graph():
    pw = _packed(300, 4096, 4, False, 128, 2)
    out = torch.empty(300, 4096, device="cuda")
    _check_graph("dequantize_groupwise", lambda: bg.dequantize_groupwise(pw, out), [out])


@pytest.mark.parametrize("b", [1, 3, 4, 8, 16])
def test_w4a16_gemv_graph(b):
    pw = _packed(1000, 4352, 4, False, 128, 3)
    x = _rand_bf16((b, 4352), 4)
    y = torch.empty(b, 1000, device="cuda")
    _check_graph(f"w4a16_gemv b={b}", lambda: bg.w4a16_gemv(x, pw, y), [y])


@pytest.mark.parametrize("b", [4, 16])
def test_w4a16_gemv_split_runs_graph(b):
    # 4096 x 10240: 32 row blocks of the shared-stage kernel, k split into 8
    # runs that add into y after the fill kernel
    pw = _packed(4096, 10240, 4, False, 128, 5)
    x = _rand_bf16((b, 10240), 6)
    y = torch.empty(b, 4096, device="cuda")
    _check_graph(f"w4a16_gemv split runs b={b}", lambda: bg.w4a16_gemv(x, pw, y), [y], rel=1e-5)


@pytest.mark.parametrize("b,n,k,rel", [(1, 1000, 4352, 0.0), (16, 2048, 8192, 1e-5)])
def test_w8a16_gemv_graph(b, n, k, rel):
    pw = _packed(n, k, 8, False, 128, 7)
    x = _rand_bf16((b, k), 8)
    y = torch.empty(b, n, device="cuda")
    _check_graph(f"w8a16_gemv b={b} {n}x{k}", lambda: bg.w8a16_gemv(x, pw, y), [y], rel=rel)


@pytest.mark.parametrize("b,n,k,rel", [(1, 1000, 4352, 0.0), (16, 2048, 8192, 1e-5)])
def test_mxfp4_graph(b, n, k, rel):
    w = _rand_bf16((n, k), 9, 0.02)
    mw = bg.mxfp4_quantize(w)
    _check_graph(f"mxfp4_quantize {n}x{k}", lambda: bg.mxfp4_quantize(w, out=mw), [mw.codes, mw.scales])
    x = _rand_bf16((b, k), 10)
    y = torch.empty(b, n, device="cuda")
    _check_graph(f"mxfp4_gemv b={b} {n}x{k}", lambda: bg.mxfp4_gemv(x, mw, y), [y], rel=rel)


def test_prefill_gemms_graph():
    n, k, m = 520, 4096, 100
    pw = _packed(n, k, 4, False, 128, 11)
    x = _rand_bf16((m, k), 12)
    y = torch.empty(m, n, device="cuda")
    _check_graph("w4a16_gemm", lambda: bg.w4a16_gemm(x, pw, y), [y])
    mw = bg.mxfp4_quantize(_rand_bf16((n, k), 13, 0.02))
    y2 = torch.empty(m, n, device="cuda")
    _check_graph("mxfp4_gemm", lambda: bg.mxfp4_gemm(x, mw, y2), [y2])


def test_smoothquant_chain_graph():
    t, n, k = 96, 512, 2048
    x = _rand_bf16((t, k), 14)
    w = _rand_bf16((n, k), 15, 0.02)
    s = torch.empty(k, device="cuda")
    _check_graph("smooth_scale", lambda: bg.smooth_scale(x, w, 0.5, s=s), [s])
    qx = torch.empty(t, k, dtype=torch.int8, device="cuda")
    sx = torch.empty(t, device="cuda")
    _check_graph("quant_per_token_int8", lambda: bg.quant_per_token_int8(x, s, qx, sx), [qx, sx])
    pw = bg.quantize_groupwise(w, 8, True, k, s)
    qw, sw = pw.codes.view(torch.int8), pw.scales.view(-1)
    y = torch.empty(t, n, device="cuda")
    acc = torch.empty(t, n, dtype=torch.int32, device="cuda")
    _check_graph("w8a8_gemm", lambda: bg.w8a8_gemm(qx, sx, qw, sw, y=y, acc=acc), [y, acc])
