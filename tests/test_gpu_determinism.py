"""Repeated calls give the same bits.

The library documents one result whose last bits may vary from call to
call: a batch 4..16 GEMV that splits k into more than two runs, which add
their partial sums into y with float atomics. Everything else is
deterministic: the GPTQ factor sums its split-k partials in a fixed order,
and a split GEMV with exactly two runs adds 0 + a + b, which is the same
float in either order. Each case below is called twice on the same inputs,
with other work between the calls, into freshly poisoned outputs, and the
outputs must agree bit for bit.
"""
import pytest
import torch

import bit_gemv_amd as bg
from gpu_helpers import say

pytestmark = pytest.mark.gpu


def _rand_bf16(shape, seed, scale=1.0):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return (torch.randn(shape, generator=g, device="cuda") * scale).to(torch.bfloat16)


def _twice(what, fn, outs):
    """fn writes outs; call it twice with unrelated work in between."""
    say(f"determinism {what}")
    for o in outs:
        o.fill_(float("nan")) if o.dtype.is_floating_point else o.fill_(77)
    fn()
    torch.cuda.synchronize()
    first = [o.clone() for o in outs]
    # unrelated device work between the calls
    junk = _rand_bf16((2048, 2048), 999)
    (junk.float() @ junk.float()).sum().item()
    for o in outs:
        o.fill_(float("nan")) if o.dtype.is_floating_point else o.fill_(77)
    fn()
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(first, outs)):
        assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                           b.view(torch.int32) if b.dtype == torch.float32 else b), \
            f"{what}: output {i} differs between two calls"


def test_gptq_factor_and_column_loop_repeat():
    t, k, n = 256, 1024, 384
    x = _rand_bf16((t, k), 1)
    w = _rand_bf16((n, k), 2, 0.02)
    u = torch.empty(k, k, device="cuda")
    _twice("gptq_hessian_factor", lambda: bg.gptq_hessian_factor(x, 0.01, u=u), [u])
    pw = bg.gptq_quantize(w, u, 4, False, 128)
    outs = [pw.codes, pw.scales, pw.zeros]

    def loop():
        q = bg.gptq_quantize(w, u, 4, False, 128)
        for o, r in zip(outs, [q.codes, q.scales, q.zeros]):
            o.copy_(r)
    _twice("gptq_quantize", loop, outs)


# 12288 x 4096 at batch 8 and 16 (INT4, MXFP4: 16 stages of 256 k): 96 row
# blocks of the shared-stage kernel, k split into two runs after the fill
# kernel
@pytest.mark.parametrize("fmt", ["int4", "mxfp4"])
@pytest.mark.parametrize("b", [8, 16])
def test_two_run_batch_gemv_repeat(fmt, b):
    n, k = 12288, 4096
    w = _rand_bf16((n, k), 3, 0.02)
    x = _rand_bf16((b, k), 4)
    y = torch.empty(b, n, device="cuda")
    if fmt == "mxfp4":
        mw = bg.mxfp4_quantize(w)
        fn = lambda: bg.mxfp4_gemv(x, mw, y)  # noqa: E731
    else:
        pw = bg.quantize_groupwise(w, 4, False, 128)
        fn = lambda: bg.w4a16_gemv(x, pw, y)  # noqa: E731
    _twice(f"{fmt} gemv b={b} {n}x{k}", fn, [y])


@pytest.mark.parametrize("b", [1, 2, 3])
def test_small_batch_gemv_repeat(b):
    # the VALU kernel (batch 1..3 always) reduces through LDS in a fixed
    # order, no atomics
    n, k = 8192, 28672
    pw = bg.quantize_groupwise(_rand_bf16((n, k), 5, 0.02), 4, False, 128)
    x = _rand_bf16((b, k), 6)
    y = torch.empty(b, n, device="cuda")
    _twice(f"w4a16_gemv b={b} {n}x{k}", lambda: bg.w4a16_gemv(x, pw, y), [y])
