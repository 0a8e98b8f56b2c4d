"""W8A16 GEMV (batch 1..16) against the oracle's fp64 result on the same INT8 codes."""
import numpy as np
import pytest

import bit_gemv_amd as bg
import oracle
from gpu_helpers import assert_close, assert_same_bits, dev_bf16, host, say
from workloads import f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def _case(n, k, b, sym, group=128, seed=0, w_scale=0.02, x_mult=None):
    rng = np.random.default_rng(seed)
    w = f32_to_bf16_bits(rng.standard_normal((n, k)) * w_scale)
    xf = rng.standard_normal((b, k))
    if x_mult is not None:
        xf = xf * x_mult
    x = f32_to_bf16_bits(xf)
    say(f"w8a16 gemv n={n} k={k} b={b} sym={sym} group={group}")
    pw = bg.quantize_groupwise(dev_bf16(w), 8, sym, group)
    c_ref, s_ref, z_ref = oracle.quantize(w, 8, sym, group)
    assert_same_bits(host(pw.codes), c_ref, "codes")
    y = host(bg.w8a16_gemv(dev_bf16(x), pw))
    y_ref = oracle.w8a16_matmul(x, c_ref, s_ref, z_ref, n, k, sym, group)
    assert_close(y, y_ref, f"y n={n} k={k} b={b}")


@pytest.mark.parametrize("sym", [False, True])
@pytest.mark.parametrize("n,k", [(1, 128), (5, 384), (67, 2048 + 128), (300, 4096), (129, 11008),
                                 (96, 8192), (33, 28672)])
def test_batch1_shapes(n, k, sym):
    """One to many chunks of 1024 k, a half-filled last chunk, ragged rows."""
    _case(n, k, 1, sym)


@pytest.mark.parametrize("sym", [False, True])
@pytest.mark.parametrize("n,k", [(16384 + 37, 2048 + 512), (20000, 8192), (8192 + 3, 16384 + 512),
                                 (4096 + 5, 4096 + 128)])
def test_tall_batch1(n, k, sym):
    """Tall matrices (8 rows per wave) with ragged rows and partial chunks."""
    _case(n, k, 1, sym, seed=n % 97)


@pytest.mark.parametrize("b", [2, 3, 4, 5, 7, 8, 9, 12, 16])
@pytest.mark.parametrize("sym", [False, True])
def test_batches(b, sym):
    """Every kernel batch width (1..4 exact, 8 and 16 with unused rows)."""
    _case(203, 4096 + 640, b, sym, seed=b)


@pytest.mark.parametrize("b", [1, 4, 8, 16])
def test_batches_tall(b):
    _case(12288 + 7, 4096, b, False, seed=b + 40)


@pytest.mark.parametrize("b", [2, 3])
@pytest.mark.parametrize("sym", [False, True])
@pytest.mark.parametrize("n,k", [(4096 + 9, 8192 + 128), (300, 9216)])
def test_small_batches_long_rows(n, k, b, sym):
    """Batch 2 and 3 on rows of 8 and more chunks: the four-way k split,
    with 8 rows a wave (4105 rows) and 4 (300 rows)."""
    _case(n, k, b, sym, seed=b + n % 13)


@pytest.mark.parametrize("b", [1, 6])
@pytest.mark.parametrize("group,k", [(256, 4096), (384, 1152 * 3), (1024, 4096), ("k", 3072), ("k", 128)])
def test_larger_groups(b, group, k):
    """Groups wider than 128, one not dividing the 1024-wide chunk (384), and
    per-channel (one group per row)."""
    _case(300, k, b, False, group=k if group == "k" else group, seed=b)


def test_activation_outlier_channels():
    k = 4096
    mult = np.ones(k)
    mult[[5, 900, 4000]] = [20.0, 40.0, 60.0]
    _case(128, k, 4, True, x_mult=mult, seed=3)


def test_extreme_codes():
    """Weights whose groups hit every end code: q = -127 / 127 (symmetric) and
    0 / 255 (asymmetric), the bytes where the unsigned conversion and the
    0x80 flip matter most."""
    rng = np.random.default_rng(7)
    n, k = 64, 2048
    w = rng.standard_normal((n, k)) * 0.02
    w[:, ::128] = 0.5
    w[:, 1::128] = -0.5
    wb = f32_to_bf16_bits(w)
    x = f32_to_bf16_bits(rng.standard_normal((3, k)))
    for sym in (False, True):
        say(f"w8a16 extreme codes sym={sym}")
        pw = bg.quantize_groupwise(dev_bf16(wb), 8, sym, 128)
        c_ref, s_ref, z_ref = oracle.quantize(wb, 8, sym, 128)
        assert_same_bits(host(pw.codes), c_ref, "codes")
        y = host(bg.w8a16_gemv(dev_bf16(x), pw))
        assert_close(y, oracle.w8a16_matmul(x, c_ref, s_ref, z_ref, n, k, sym, 128), f"extreme sym={sym}")


# Batch 4 from about 40M weights with k >= 8192, 5..8 from 40M and 9..16
# from 16M go to the shared-stage kernel: 128-row blocks (ragged here), k in 128-wide stages
# split into runs (uneven, some empty) whose partial sums meet in y.
@pytest.mark.parametrize("b", [5, 8, 9, 16])
@pytest.mark.parametrize("n,k", [(16384 + 33, 4096 + 384),   # 8 runs of 5 stages, the last empty
                                 (4096 + 17, 11008),         # 16 runs of 6, one with 2, one empty
                                 (8192 + 100, 8192 - 128),   # 8 runs of 8, the last with 7
                                 (40000 + 77, 2048 + 128)])  # no split
def test_shared_stage_batches(n, k, b):
    _case(n, k, b, False, seed=n % 83 + b)


@pytest.mark.parametrize("sym", [False, True])
@pytest.mark.parametrize("n,k", [(4096 + 17, 11008),       # 16 runs of 6 stages, one with 2, one empty
                                 (8192 + 100, 8192 + 256)])  # 16 runs of 5, one with 1, two empty
def test_shared_stage_batch4(n, k, sym):
    """Batch 4 goes to the shared-stage kernel (4 staged activation rows)
    from 40M weights where k >= 8192."""
    _case(n, k, 4, sym, seed=n % 71)


@pytest.mark.parametrize("b", [6, 12])
@pytest.mark.parametrize("n,k", [(16384 + 33, 4096 + 384), (4096, 4096)])
def test_shared_stage_symmetric(n, k, b):
    """Symmetric int8 codes (the 0x80 flip and the constant 128); 4096 x 4096
    takes the shared-stage kernel only at batch 9 and more."""
    _case(n, k, b, True, seed=n % 79 + b)


@pytest.mark.parametrize("group", [256, 1024, "k"])
def test_shared_stage_larger_groups(group):
    n, k = 10240 + 3, 8192
    _case(n, k, 16, False, group=k if group == "k" else group, seed=7)


def test_shared_stage_extreme_codes():
    """End codes (-127 / 127, 0 / 255) through the shared-stage conversion."""
    rng = np.random.default_rng(8)
    n, k = 10240 + 3, 4096
    w = rng.standard_normal((n, k)) * 0.02
    w[:, ::128] = 0.5
    w[:, 1::128] = -0.5
    wb = f32_to_bf16_bits(w)
    x = f32_to_bf16_bits(rng.standard_normal((16, k)))
    for sym in (False, True):
        say(f"w8a16 shared-stage extreme codes sym={sym}")
        pw = bg.quantize_groupwise(dev_bf16(wb), 8, sym, 128)
        c_ref, s_ref, z_ref = oracle.quantize(wb, 8, sym, 128)
        y = host(bg.w8a16_gemv(dev_bf16(x), pw))
        assert_close(y, oracle.w8a16_matmul(x, c_ref, s_ref, z_ref, n, k, sym, 128), f"extreme sym={sym}")


def test_int4_codes_are_refused():
    import torch
    w = torch.zeros((8, 256), dtype=torch.bfloat16, device="cuda")
    pw = bg.quantize_groupwise(w, 4, True, 128)
    x = torch.zeros((1, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        bg.w8a16_gemv(x, pw)


def test_batch_over_16_is_unsupported():
    import torch
    w = torch.zeros((8, 256), dtype=torch.bfloat16, device="cuda")
    pw = bg.quantize_groupwise(w, 8, True, 128)
    x = torch.zeros((17, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(bg.LibquantError) as e:
        bg.w8a16_gemv(x, pw)
    assert e.value.status == bg.LQ_ERR_UNSUPPORTED
