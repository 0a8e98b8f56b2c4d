"""The allocation-free GPTQ column loop (gptq_quantize_noalloc, scratch in the
library's static device array) against gptq_quantize with a caller
workspace: codes, scales and zeros bit for bit, on two calls in a row, the
second with a smaller matrix, so the second call runs on scratch the first
one left behind."""
import ctypes

import numpy as np
import pytest
import torch

import bit_gemv_amd as bg
from gpu_helpers import assert_same_bits, dev_bf16, host, say
from workloads import WORKLOADS, f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def _inputs(t, n, k, seed):
    rng = np.random.default_rng(seed)
    x = f32_to_bf16_bits(rng.standard_normal((t, k)))
    w = f32_to_bf16_bits(rng.standard_normal((n, k)) * 0.02)
    return x, w


def _both(w, u, bits, symmetric, group, what):
    n, k = w.shape
    say(f"gptq_quantize_noalloc {what}: n={n} k={k} bits={bits} sym={symmetric} group={group}")
    wd = dev_bf16(w)
    ref = bg.gptq_quantize(wd, u, bits, symmetric, group)
    got = bg.gptq_quantize_noalloc(wd, u, bits, symmetric, group)
    assert_same_bits(host(got.codes), host(ref.codes), f"{what} codes")
    assert_same_bits(host(got.scales), host(ref.scales), f"{what} scales")
    if not symmetric:
        assert_same_bits(host(got.zeros), host(ref.zeros), f"{what} zeros")


def test_two_calls_in_a_row_second_smaller():
    lib = bg.load_library()
    assert lib.gptq_quantize_noalloc_max_bytes() == 72 << 20
    wl = WORKLOADS["awq7b"]
    # 1: the 7B q projection (4096 x 4096, 66 MiB of scratch), 512 calibration tokens
    x = wl.activation(4096, wl.tokens)
    u = bg.gptq_hessian_factor(dev_bf16(x))
    _both(wl.weight(0, 0), u, 4, False, 128, "q projection")
    # 2: a smaller, ragged matrix on the scratch the first call left behind
    x2, w2 = _inputs(96, 300, 1024, seed=3)
    u2 = bg.gptq_hessian_factor(dev_bf16(x2))
    _both(w2, u2, 4, True, 128, "300 x 1024")
    _both(w2, u2, 8, False, 256, "300 x 1024 INT8 G=256")


def test_rejects_more_scratch_than_it_holds():
    lib = bg.load_library()
    P = ctypes.c_void_p
    # 4096 x 4608 needs 72 MiB + 2 MiB: rejected before any work
    st = lib.gptq_quantize_noalloc(P(1 << 20), 4096, 4608, P(2 << 20), 4, 0, 128, P(3 << 20), P(4 << 20),
                                   P(5 << 20), None)
    assert st == bg.LQ_ERR_UNSUPPORTED
    assert b"static scratch" in lib.lq_last_error()
