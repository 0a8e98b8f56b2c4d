"""MXFP4 quantizer (bit-exact) and MXFP4 x bf16 GEMV (fp64 oracle) on the GPU."""
import numpy as np
import pytest

import bit_gemv_amd as bg
import oracle
from gpu_helpers import assert_close, assert_same_bits, dev_bf16, host, say
from workloads import WORKLOADS, f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def _quant_check(w, what):
    n, k = w.shape
    say(f"mxfp4_quantize {what} n={n} k={k}")
    mw = bg.mxfp4_quantize(dev_bf16(w))
    c_ref, s_ref = oracle.mx_quantize(w)
    assert_same_bits(host(mw.scales), s_ref, f"{what} scales")
    assert_same_bits(host(mw.codes), c_ref, f"{what} codes")
    return mw, c_ref, s_ref


@pytest.mark.parametrize("n,k", [(1, 128), (7, 384), (300, 4096), (4096 + 3, 11008)])
def test_quantize_random_rows(n, k):
    """Rows spread over 2^-40 .. 2^40 so blocks take many exponents."""
    rng = np.random.default_rng(n + k)
    w = rng.standard_normal((n, k)) * np.exp(rng.uniform(-28, 28, (n, 1)))
    _quant_check(f32_to_bf16_bits(w), "random")


def test_quantize_every_finite_bf16_value():
    """All finite bf16 bit patterns, in order, 32 to a block (each block holds
    neighbouring patterns, so every value meets scales near its own), plus the
    same patterns shuffled across blocks."""
    pats = np.arange(65536, dtype=np.uint32)
    exp = (pats >> 7) & 0xFF
    finite = pats[exp != 0xFF].astype(np.uint16)
    pad = (-finite.size) % 4096
    allv = np.concatenate([finite, np.zeros(pad, np.uint16)]).reshape(-1, 4096)
    _quant_check(allv, "every bf16 (ordered)")
    rng = np.random.default_rng(5)
    _quant_check(rng.permutation(allv.ravel()).reshape(allv.shape), "every bf16 (shuffled)")


def test_quantize_ties_zeros_and_tiny_blocks():
    rng = np.random.default_rng(6)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    rows = []
    for e in (-127, -126, -20, 0, 13, 120):
        r = np.zeros(128)
        r[0] = 6.0
        r[1:8], r[8:15] = mids, -mids
        r[32:64] = rng.choice([0.5, 1.0, 1.5, 3.0, 6.0], 32) * rng.choice([-1, 1], 32)
        r[64] = 6.0
        r[96:128] = 0.0                                # an all-zero block
        rows.append(np.ldexp(r, e))
    w = f32_to_bf16_bits(np.array(rows, np.float32))
    w[0, 100] = 0x8000                                 # -0.0 in the zero block
    w[1, 101] = 0x0001                                 # the smallest subnormal bf16
    _quant_check(w, "ties/zeros")


def _gemv_case(n, k, b, seed, what=""):
    rng = np.random.default_rng(seed)
    w = f32_to_bf16_bits(rng.standard_normal((n, k)) * 0.02)
    x = f32_to_bf16_bits(rng.standard_normal((b, k)))
    mw, c_ref, s_ref = _quant_check(w, f"gemv {what}")
    say(f"mxfp4_gemv n={n} k={k} b={b}")
    y = host(bg.mxfp4_gemv(dev_bf16(x), mw))
    assert_close(y, oracle.mx_matmul(x, c_ref, s_ref, n, k), f"mx y n={n} k={k} b={b}")


@pytest.mark.parametrize("n,k", [(1, 128), (5, 384), (67, 2048 + 128), (300, 4096), (129, 11008), (33, 28672),
                                 (16384 + 37, 2048 + 512), (8192 + 3, 16384 + 512), (4096, 9216)])
def test_gemv_batch1(n, k):
    """One to many chunks of 2048 k, partial last chunks, ragged rows, and
    tall matrices (8 rows per wave)."""
    _gemv_case(n, k, 1, seed=n % 97)


@pytest.mark.parametrize("b", [2, 3, 4, 5, 8, 9, 16])
def test_gemv_batches(b):
    _gemv_case(203, 4096 + 640, b, seed=b)


def test_gemv_batch_over_16_is_unsupported():
    import torch
    mw = bg.mxfp4_quantize(torch.zeros((8, 256), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(bg.LibquantError) as e:
        bg.mxfp4_gemv(torch.zeros((17, 256), dtype=torch.bfloat16, device="cuda"), mw)
    assert e.value.status == bg.LQ_ERR_UNSUPPORTED


def test_workload_gate_up_sampled_rows():
    """The 70B-shaped gate|up matrix (57344 x 8192) at full size: sampled
    rows of the codes and scales bit-exact, and the batch-1 outputs of those
    rows against the oracle one by one."""
    wl = WORKLOADS["llama70b_decode"]
    import torch
    w = torch.cat([dev_bf16(wl.weight(0, i)) for i in (4, 5)], 0)
    n, k = w.shape
    say(f"mxfp4 gate|up {n}x{k}")
    mw = bg.mxfp4_quantize(w)
    x = wl.activation(k, 1)
    y = host(bg.mxfp4_gemv(dev_bf16(x), mw))
    rows = np.sort(np.random.default_rng(1).choice(n, 48, replace=False))
    wr = host(w[torch.from_numpy(rows).cuda()].view(torch.int16)).view(np.uint16)
    c_ref, s_ref = oracle.mx_quantize(wr)
    assert_same_bits(host(mw.codes)[rows], c_ref, "sampled codes")
    assert_same_bits(host(mw.scales)[rows], s_ref, "sampled scales")
    assert_close(y[:, rows], oracle.mx_matmul(x, c_ref, s_ref, rows.size, k), "sampled y")


# Batch 4..8 from about 40M weights and 9..16 from 16M go to the
# shared-stage kernel, which folds each block's scale into the E2M1 -> bf16
# conversion: ragged 128-row blocks, half last 256-wide stages, runs of k
# (some empty), 4, 8 or 16 staged batch rows.
@pytest.mark.parametrize("b", [4, 5, 8, 9, 16])
@pytest.mark.parametrize("n,k", [(16384 + 33, 4096 + 384), (4096 + 17, 11008), (1000, 45056),
                                 (40000 + 77, 2048 + 128)])
def test_shared_stage_batches(n, k, b):
    _gemv_case(n, k, b, seed=n % 71 + b, what="shared")


@pytest.mark.parametrize("b", [9, 16])
def test_shared_stage_from_16m_weights(b):
    _gemv_case(4096, 4096, b, seed=b, what="shared 4096")


@pytest.mark.parametrize("b", [5, 16])
def test_shared_stage_row_magnitudes(b):
    """Rows scaled by 2^-130 .. 2^90: block scales over most of the E8M0
    range, and at the low end elements that are bf16 subnormals once scaled
    (the conversion with the block scale and the MFMA keep them). Each
    output is checked against its own magnitude, sum_j |x_j w_hat_j|."""
    n, k = 10240 + 3, 4096
    rng = np.random.default_rng(20 + b)
    e = rng.integers(-130, 91, n)
    w = f32_to_bf16_bits(rng.standard_normal((n, k)) * np.ldexp(1.0, e)[:, None])
    x = f32_to_bf16_bits(rng.standard_normal((b, k)))
    mw, c_ref, s_ref = _quant_check(w, "row magnitudes")
    say(f"mxfp4_gemv row magnitudes n={n} k={k} b={b}")
    y = host(bg.mxfp4_gemv(dev_bf16(x), mw)).astype(np.float64)
    y_ref = oracle.mx_matmul(x, c_ref, s_ref, n, k)
    from workloads import bf16_bits_to_f32
    bound = np.abs(bf16_bits_to_f32(x).astype(np.float64)) @ np.abs(oracle.mx_dequantize(c_ref, s_ref, n, k)).T
    err = np.abs(y - y_ref)
    worst = float(np.max(err / np.where(bound > 0, bound, 1.0)))
    say(f"  worst |y - y_ref| / sum|x w| = {worst:.2e}")
    assert np.all(np.isfinite(y))
    assert np.all(err <= 1e-4 * bound), worst


# --------------------------------------------------------------------------
# MXFP4 prefill GEMM (bf16 MFMA on E2M1 * 2^e operands converted exactly)

def _gemm_case(m, n, k, seed, w_scale=None, x_mult=None, what=""):
    rng = np.random.default_rng(seed)
    wf = rng.standard_normal((n, k)) * 0.02
    if w_scale is not None:
        wf = wf * w_scale
    w = f32_to_bf16_bits(wf)
    xf = rng.standard_normal((m, k))
    if x_mult is not None:
        xf = xf * x_mult
    x = f32_to_bf16_bits(xf)
    mw, c_ref, s_ref = _quant_check(w, f"gemm {what}")
    say(f"mxfp4_gemm m={m} n={n} k={k} {what}")
    y = host(bg.mxfp4_gemm(dev_bf16(x), mw))
    y_ref = oracle.mx_matmul(x, c_ref, s_ref, n, k)
    assert_close(y, y_ref, f"mx gemm m={m} n={n} k={k} {what}")
    return y, y_ref


@pytest.mark.parametrize("m,n,k", [(1, 16, 128), (5, 33, 384), (64, 200, 1024), (130, 130, 2048 + 128),
                                   (257, 96, 4096), (128, 128, 128), (300, 1030, 2048)])
def test_gemm_shapes(m, n, k):
    """Single and several 128 x 128 tiles, ragged rows and columns (partial
    tiles whose loads read zeros), one to 32 steps of k, n a multiple of
    8 tiles (the XCD-grouped tile order) and not."""
    _gemm_case(m, n, k, seed=m + n + k)


def test_gemm_outlier_channels():
    k = 2048
    mult = np.ones(k)
    mult[[3, 500, 1500, 2047]] = [20.0, 35.0, 50.0, 60.0]
    _gemm_case(200, 144, k, seed=9, x_mult=mult, what="outliers")


def test_gemm_row_magnitudes():
    """Rows of W scaled by 2^-130 .. 2^90: block scales over most of the E8M0
    range, with bf16-subnormal operands at the low end (the scaled conversion
    and the MFMA keep them). Each output is checked against its own
    magnitude, sum_j |x_j w_hat_j|."""
    m, n, k = 70, 1000 + 3, 1024
    rng = np.random.default_rng(77)
    e = rng.integers(-130, 91, n)
    w = f32_to_bf16_bits(rng.standard_normal((n, k)) * np.ldexp(1.0, e)[:, None])
    x = f32_to_bf16_bits(rng.standard_normal((m, k)))
    mw, c_ref, s_ref = _quant_check(w, "gemm row magnitudes")
    say(f"mxfp4_gemm row magnitudes m={m} n={n} k={k}")
    y = host(bg.mxfp4_gemm(dev_bf16(x), mw)).astype(np.float64)
    y_ref = oracle.mx_matmul(x, c_ref, s_ref, n, k)
    from workloads import bf16_bits_to_f32
    bound = np.abs(bf16_bits_to_f32(x).astype(np.float64)) @ np.abs(oracle.mx_dequantize(c_ref, s_ref, n, k)).T
    err = np.abs(y - y_ref)
    worst = float(np.max(err / np.where(bound > 0, bound, 1.0)))
    say(f"  worst |y - y_ref| / sum|x w| = {worst:.2e}")
    assert np.all(np.isfinite(y))
    assert np.all(err <= 1e-4 * bound), worst


def test_gemv_and_gemm_agree():
    rng = np.random.default_rng(12)
    n, k = 300, 4096
    w = f32_to_bf16_bits(rng.standard_normal((n, k)) * 0.02)
    x = f32_to_bf16_bits(rng.standard_normal((16, k)))
    mw = bg.mxfp4_quantize(dev_bf16(w))
    yv = host(bg.mxfp4_gemv(dev_bf16(x), mw))
    ym = host(bg.mxfp4_gemm(dev_bf16(x), mw))
    assert np.abs(yv - ym).max() <= 1e-4 * np.abs(ym).max()


def test_gemm_k_not_a_multiple_of_128_is_unsupported():
    import torch
    # a 160-wide MXFP4 weight (5 blocks of 32): valid MX, not a k this GEMM takes
    mw = bg.MxWeight(torch.zeros((8, 80), dtype=torch.uint8, device="cuda"),
                     torch.zeros((8, 5), dtype=torch.uint8, device="cuda"), 8, 160)
    with pytest.raises(bg.LibquantError) as e:
        bg.mxfp4_gemm(torch.zeros((4, 160), dtype=torch.bfloat16, device="cuda"), mw)
    assert e.value.status == bg.LQ_ERR_UNSUPPORTED


@pytest.mark.parametrize("idx", [0, 1, 2])
def test_gemm_prefill_workload_sampled(idx):
    """The M = 2048 prefill shapes (8192 x 8192, 28672 x 8192, 8192 x 28672)
    at full size with the workload's outlier activations; outputs on a
    seeded sample of rows and columns against the oracle, and all finite."""
    pf = WORKLOADS["prefill70b"]
    lin = pf.linears[idx]
    say(f"mxfp4_gemm prefill70b {lin.name} {lin.n}x{lin.k} M={pf.tokens}")
    w = pf.weight(0, idx)
    x = pf.activation(lin.k, pf.tokens)
    mw = bg.mxfp4_quantize(dev_bf16(w))
    y = host(bg.mxfp4_gemm(dev_bf16(x), mw))
    rng = np.random.default_rng(200 + idx)
    rows = np.sort(rng.choice(pf.tokens, 24, replace=False))
    cols = np.sort(rng.choice(lin.n, 48, replace=False))
    c_ref, s_ref = oracle.mx_quantize(w[cols])
    assert_same_bits(host(mw.codes)[cols], c_ref, "codes (sampled rows)")
    assert_same_bits(host(mw.scales)[cols], s_ref, "scales (sampled rows)")
    y_ref = oracle.mx_matmul(x[rows], c_ref, s_ref, cols.size, lin.k)
    assert_close(y[np.ix_(rows, cols)], y_ref, f"mx prefill {lin.name} sampled")
    assert np.all(np.isfinite(y))
