"""W4A16 prefill GEMM (bf16 MFMA) against the oracle's fp64 result on the same codes."""
import numpy as np
import pytest

import bit_gemv_amd as bg
import oracle
from gpu_helpers import assert_close, assert_same_bits, dev_bf16, host, say
from workloads import WORKLOADS, f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def _case(m, n, k, sym, group=128, seed=0, x_mult=None):
    rng = np.random.default_rng(seed)
    w = f32_to_bf16_bits(rng.standard_normal((n, k)) * 0.02)
    xf = rng.standard_normal((m, k))
    if x_mult is not None:
        xf = xf * x_mult
    x = f32_to_bf16_bits(xf)
    say(f"gemm m={m} n={n} k={k} sym={sym} group={group}")
    pw = bg.quantize_groupwise(dev_bf16(w), 4, sym, group)
    c_ref, s_ref, z_ref = oracle.quantize(w, 4, sym, group)
    assert_same_bits(host(pw.codes), c_ref, "codes")
    y = host(bg.w4a16_gemm(dev_bf16(x), pw))
    y_ref = oracle.w4a16_matmul(x, c_ref, s_ref, z_ref, n, k, sym, group)
    assert_close(y, y_ref, f"Y m={m} n={n} k={k}")


@pytest.mark.parametrize("sym", [False, True])
@pytest.mark.parametrize("m,n,k", [(1, 16, 128), (5, 33, 384), (64, 200, 1024), (130, 130, 2048 + 128),
                                   (257, 96, 4096), (128, 128, 128)])
def test_shapes(m, n, k, sym):
    _case(m, n, k, sym, seed=m + n)


@pytest.mark.parametrize("group", [256, "k"])
def test_larger_groups(group):
    _case(96, 160, 1024, False, group=1024 if group == "k" else group, seed=7)


def test_outlier_channels():
    k = 2048
    mult = np.ones(k)
    mult[[3, 500, 1500, 2047]] = [20.0, 35.0, 50.0, 60.0]
    _case(200, 144, k, False, x_mult=mult, seed=9)


def test_gemv_and_gemm_agree():
    """Batch 1..16 through both entry points: same definition, fp32 sums."""
    rng = np.random.default_rng(11)
    n, k = 300, 4096
    w = f32_to_bf16_bits(rng.standard_normal((n, k)) * 0.02)
    x = f32_to_bf16_bits(rng.standard_normal((16, k)))
    pw = bg.quantize_groupwise(dev_bf16(w), 4, False, 128)
    yv = host(bg.w4a16_gemv(dev_bf16(x), pw))
    ym = host(bg.w4a16_gemm(dev_bf16(x), pw))
    assert np.abs(yv - ym).max() <= 1e-4 * np.abs(ym).max()


@pytest.mark.parametrize("idx", [0, 1, 2])
def test_prefill_workload_sampled(idx):
    """The M = 2048 prefill shapes at full size; outputs checked on a seeded
    sample of rows and columns (the oracle computes them one by one)."""
    pf = WORKLOADS["prefill70b"]
    lin = pf.linears[idx]
    say(f"gemm prefill70b {lin.name} {lin.n}x{lin.k} M={pf.tokens}")
    w = pf.weight(0, idx)
    x = pf.activation(lin.k, pf.tokens)
    pw = bg.quantize_groupwise(dev_bf16(w), 4, pf.symmetric, pf.group)
    y = host(bg.w4a16_gemm(dev_bf16(x), pw))
    rng = np.random.default_rng(100 + idx)
    rows = np.sort(rng.choice(pf.tokens, 24, replace=False))
    cols = np.sort(rng.choice(lin.n, 48, replace=False))
    c_ref, s_ref, z_ref = oracle.quantize(w[cols], 4, pf.symmetric, pf.group)
    assert_same_bits(host(pw.codes)[cols], c_ref, "codes (sampled rows)")
    y_ref = oracle.w4a16_matmul(x[rows], c_ref, s_ref, z_ref, cols.size, lin.k, pf.symmetric, pf.group)
    assert_close(y[np.ix_(rows, cols)], y_ref, f"prefill {lin.name} sampled")
    assert np.all(np.isfinite(y))
