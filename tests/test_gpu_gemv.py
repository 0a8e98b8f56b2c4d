"""W4A16 GEMV (batch 1..16) against the oracle's fp64 result on the same codes."""
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
    say(f"gemv n={n} k={k} b={b} sym={sym} group={group}")
    pw = bg.quantize_groupwise(dev_bf16(w), 4, sym, group)
    c_ref, s_ref, z_ref = oracle.quantize(w, 4, sym, group)
    assert_same_bits(host(pw.codes), c_ref, "codes")
    y = host(bg.w4a16_gemv(dev_bf16(x), pw))
    y_ref = oracle.w4a16_matmul(x, c_ref, s_ref, z_ref, n, k, sym, group)
    assert_close(y, y_ref, f"y n={n} k={k} b={b}")


@pytest.mark.parametrize("sym", [False, True])
@pytest.mark.parametrize("n,k", [(1, 128), (5, 384), (67, 2048 + 128), (300, 4096), (129, 11008),
                                 (96, 8192), (33, 28672), (40, 9728), (61, 10368), (1001, 14336)])
def test_batch1_shapes(n, k, sym):
    _case(n, k, 1, sym)


@pytest.mark.parametrize("sym", [False, True])
@pytest.mark.parametrize("n,k", [(16384 + 37, 2048 + 512), (20000, 8192), (32768 + 5, 4096), (16400, 512),
                                 (8192 + 3, 16384 + 512), (3001, 28672), (12000 + 7, 4096 + 128)])
def test_tall_batch1(n, k, sym):
    """Tall matrices and long rows (4 or 8 rows per wave, k split 1, 2 or 4
    ways across the block's waves, staged and per-row scale loads), with
    ragged rows and a partial last chunk."""
    _case(n, k, 1, sym, seed=n % 97)


@pytest.mark.parametrize("b", [2, 3, 4, 5, 7, 8, 11, 16])
@pytest.mark.parametrize("sym", [False, True])
def test_batches(b, sym):
    _case(203, 4096 + 640, b, sym, seed=b)


@pytest.mark.parametrize("b", [5, 16])
@pytest.mark.parametrize("sym", [False, True])
@pytest.mark.parametrize("n,k", [(4096 + 17, 4096), (8192, 4096), (33, 128), (1000, 128 * 37), (64, 28672),
                                 (12288 + 5, 2048 + 128), (16384 + 33, 2048 + 128), (20000, 2048)])
def test_mfma_batches(n, k, b, sym):
    """Batches 5..16 below about 40M weights: the LDS-ring kernel (n up to
    12288: ragged 16-row tiles, a half last 256-wide stage, waves with no
    stage) and the register-streaming kernel for taller matrices (ragged
    tiles, uneven group runs)."""
    _case(n, k, b, sym, seed=n % 89 + b)


# (n, k): blocks of 128 rows x runs of 256-wide stages in the shared-stage
# kernel (batch 4..16 from about 40M weights)
SHARED_SHAPES = [
    (16384 + 33, 4096 + 384),   # ragged rows, half last stage, 4 runs of 5 stages, the last with 3
    (4096 + 17, 11008),         # 4 runs of 11 stages, the last with 10
    (1000, 45056),              # 32 runs of 6 stages: one with 2, the last two empty
    (8192 + 100, 8192 - 128),   # 8 runs of 4 stages, half last stage
    (12288, 4096),              # 2 runs, whole blocks and stages
    (40000 + 77, 2048 + 128),   # 314 blocks: no split, half last stage
]


@pytest.mark.parametrize("b", [4, 5, 8, 9, 16])
@pytest.mark.parametrize("n,k", SHARED_SHAPES)
def test_shared_stage_batches(n, k, b):
    """Batch rows staged 4, 8 or 16 at a time (rows past the batch read
    zeros), asymmetric; split runs add into y through atomics."""
    _case(n, k, b, False, seed=n % 83 + b)


@pytest.mark.parametrize("b", [4, 12])
@pytest.mark.parametrize("n,k", [(16384 + 33, 4096 + 384), (1000, 45056), (40000 + 77, 2048 + 128)])
def test_shared_stage_symmetric(n, k, b):
    _case(n, k, b, True, seed=n % 79 + b)


@pytest.mark.parametrize("group", [256, 1024, "k"])
def test_shared_stage_larger_groups(group):
    """A group spans both halves of a stage (or several stages); each half
    reads its own group's scale."""
    n, k = 10240 + 3, 8192
    _case(n, k, 16, False, group=k if group == "k" else group, seed=7)


@pytest.mark.parametrize("b", [6, 16])
@pytest.mark.parametrize("group", [256, 1024, "k"])
def test_mfma_larger_groups(b, group):
    k = 4096
    _case(300, k, b, False, group=k if group == "k" else group, seed=b)


@pytest.mark.parametrize("group", [256, "k"])
def test_larger_groups(group):
    k = 2048
    _case(77, k, 3, False, group=k if group == "k" else group)


@pytest.mark.parametrize("group", [256, "k"])
def test_larger_groups_eight_way_split(group):
    # batch 1 with 5..7 chunks of 2048 runs on 8-wave blocks
    k = 11008 if group == 256 else 12288
    _case(77, k, 1, True, group=k if group == "k" else group)


def test_activation_outlier_channels():
    k = 4096
    mult = np.ones(k)
    mult[[5, 900, 4000]] = [20.0, 40.0, 60.0]
    _case(128, k, 4, False, x_mult=mult, seed=3)


def test_full_4096_square_batch1_asym():
    """The 4096 x 4096 asymmetric INT4 single-matrix workload, every output."""
    from workloads import WORKLOADS
    wl = WORKLOADS["single_4096"]
    w = wl.weight(0, 0)
    x = wl.activation(4096, 1)
    say("gemv single_4096 full")
    pw = bg.quantize_groupwise(dev_bf16(w), 4, False, 128)
    c_ref, s_ref, z_ref = oracle.quantize(w, 4, False, 128)
    assert_same_bits(host(pw.codes), c_ref, "codes")
    assert_same_bits(host(pw.scales), s_ref, "scales")
    assert_same_bits(host(pw.zeros), z_ref, "zeros")
    y = host(bg.w4a16_gemv(dev_bf16(x), pw))
    y_ref = oracle.w4a16_matmul(x, c_ref, s_ref, z_ref, 4096, 4096, False, 128)
    assert_close(y, y_ref, "single_4096 y")


def test_batch_over_16_is_unsupported():
    import torch
    w = torch.zeros((8, 256), dtype=torch.bfloat16, device="cuda")
    pw = bg.quantize_groupwise(w, 4, True, 128)
    x = torch.zeros((17, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(bg.LibquantError) as e:
        bg.w4a16_gemv(x, pw)
    assert e.value.status == bg.LQ_ERR_UNSUPPORTED


@pytest.mark.parametrize("n,k,runs", [(12288, 4096, 2), (1000, 45056, 32)])
def test_shared_stage_overwrites_y(n, k, runs):
    """Split runs add into y after it is zeroed on the same stream: a y full
    of NaN is overwritten, and a second call into the same y gives the same
    result (bit for bit with two runs, where 0 + a + b does not depend on
    the order; to rounding with more)."""
    import torch
    rng = np.random.default_rng(n + k)
    w = f32_to_bf16_bits(rng.standard_normal((n, k)) * 0.02)
    x = f32_to_bf16_bits(rng.standard_normal((16, k)))
    say(f"gemv shared-stage y overwrite n={n} k={k} runs={runs}")
    pw = bg.quantize_groupwise(dev_bf16(w), 4, False, 128)
    c_ref, s_ref, z_ref = oracle.quantize(w, 4, False, 128)
    y_ref = oracle.w4a16_matmul(x, c_ref, s_ref, z_ref, n, k, False, 128)
    y = torch.full((16, n), float("nan"), dtype=torch.float32, device="cuda")
    xd = dev_bf16(x)
    first = host(bg.w4a16_gemv(xd, pw, y)).copy()
    assert_close(first, y_ref, "first call")
    second = host(bg.w4a16_gemv(xd, pw, y))
    assert_close(second, y_ref, "second call")
    if runs == 2:
        assert np.array_equal(first.view(np.uint32), second.view(np.uint32))
