"""W8A8 INT8 GEMM: int32 accumulators bit-exact, fp32 output within tolerance,
and the whole SmoothQuant chain against the oracle's own chain."""
import numpy as np
import pytest
import torch

import bit_gemv_amd as bg
import oracle
from gpu_helpers import assert_close, assert_same_bits, dev, dev_bf16, host, say
from workloads import WORKLOADS

pytestmark = pytest.mark.gpu


def _run(qx, sx, qw, sw):
    y, acc = bg.w8a8_gemm(dev(qx), dev(sx), dev(qw), dev(sw), want_acc=True)
    return host(y), host(acc)


@pytest.mark.parametrize("m,n,k", [(1, 16, 128), (5, 33, 384), (64, 200, 1024), (130, 130, 2048 + 128),
                                   (257, 96, 4096), (128, 128, 128)])
def test_random_int8(m, n, k):
    rng = np.random.default_rng(m * 7 + n)
    qx = rng.integers(-128, 128, (m, k), dtype=np.int8)
    qw = rng.integers(-128, 128, (n, k), dtype=np.int8)
    sx = rng.uniform(1e-3, 1, m).astype(np.float32)
    sw = rng.uniform(1e-3, 1, n).astype(np.float32)
    say(f"w8a8 m={m} n={n} k={k}")
    y, acc = _run(qx, sx, qw, sw)
    acc_ref, y_ref = oracle.w8a8_gemm(qx, sx, qw, sw)
    assert_same_bits(acc, acc_ref, "acc")
    assert_close(y, y_ref, "y")


def test_extreme_accumulators():
    """Largest magnitudes: +-127 and -128 over the longest k the ABI accepts
    for a short test (every product at its maximum)."""
    k = 16384
    qx = np.full((3, k), 127, np.int8)
    qx[1] = -128
    qx[2, ::2] = -128
    qw = np.full((4, k), -128, np.int8)
    qw[1] = 127
    qw[2, 1::2] = 127
    sx = np.ones(3, np.float32)
    sw = np.ones(4, np.float32)
    say("w8a8 extremes")
    y, acc = _run(qx, sx, qw, sw)
    acc_ref, _ = oracle.w8a8_gemm(qx, sx, qw, sw)
    assert_same_bits(acc, acc_ref, "acc")


def test_no_acc_output():
    rng = np.random.default_rng(3)
    qx = rng.integers(-127, 128, (40, 512), dtype=np.int8)
    qw = rng.integers(-127, 128, (70, 512), dtype=np.int8)
    sx = rng.uniform(0.1, 1, 40).astype(np.float32)
    sw = rng.uniform(0.1, 1, 70).astype(np.float32)
    y, acc = bg.w8a8_gemm(dev(qx), dev(sx), dev(qw), dev(sw))
    assert acc is None
    _, y_ref = oracle.w8a8_gemm(qx, sx, qw, sw)
    assert_close(host(y), y_ref, "y (no acc)")


def test_smoothquant_chain_full_size():
    """The 512 x 8192 SmoothQuant workload end to end: smoothing factors,
    per-channel INT8 weights, per-token INT8 activations bit-exact in full;
    int32 accumulators and outputs on a seeded sample of (token, channel)
    pairs from the oracle's own chain."""
    sq = WORKLOADS["smoothquant"]
    lin = sq.linears[0]
    alpha = sq.extra["alpha"]
    x = sq.activation(lin.k, sq.tokens)
    w = sq.weight(0, 0)
    say("smoothquant chain 512x8192x8192")
    s_gpu = bg.smooth_scale(dev_bf16(x), dev_bf16(w), alpha)
    pw = bg.quantize_groupwise(dev_bf16(w), 8, True, lin.k, s_gpu)
    qx, sx = bg.quant_per_token_int8(dev_bf16(x), s_gpu)
    y, acc = bg.w8a8_gemm(qx, sx, pw.codes.view(torch.int8), pw.scales.view(-1), want_acc=True)
    s_ref = oracle.smooth_scale(x, w, alpha)
    assert_same_bits(host(s_gpu), s_ref, "s")
    qw_ref, sw_ref, _ = oracle.quantize(w, 8, True, lin.k, s_ref)
    assert_same_bits(host(pw.codes), qw_ref, "qw")
    assert_same_bits(host(pw.scales), sw_ref, "sw")
    qx_ref, sx_ref = oracle.quant_per_token_int8(x, s_ref)
    assert_same_bits(host(qx), qx_ref, "qx")
    assert_same_bits(host(sx), sx_ref, "sx")
    rng = np.random.default_rng(5)
    rows = np.sort(rng.choice(sq.tokens, 32, replace=False))
    cols = np.sort(rng.choice(lin.n, 64, replace=False))
    acc_ref, y_ref = oracle.w8a8_gemm(qx_ref[rows], sx_ref[rows], qw_ref.view(np.int8)[cols], sw_ref[cols, 0])
    assert_same_bits(host(acc)[np.ix_(rows, cols)], acc_ref, "acc (sampled)")
    assert_close(host(y)[np.ix_(rows, cols)], y_ref, "y (sampled)")
    # and the smoothed product stays close to the unquantized one
    xf = (x.astype(np.uint32) << 16).view(np.float32)[rows].astype(np.float64)
    wf = (w.astype(np.uint32) << 16).view(np.float32)[cols].astype(np.float64)
    full = xf @ wf.T
    rel = np.linalg.norm(host(y)[np.ix_(rows, cols)] - full) / np.linalg.norm(full)
    assert rel < 0.05, rel
