"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (fused q|k|v and gate|up matrices, batch-1 decode), on
seeded samples of rows the oracle computes one by one."""
import numpy as np
import pytest
import torch

import bit_gemv_amd as bg
import oracle
from gpu_helpers import assert_close, assert_same_bits, dev_bf16, host, say
from workloads import WORKLOADS

pytestmark = pytest.mark.gpu

GROUPS = [[0, 1, 2], [3], [4, 5], [6]]  # q|k|v, o, gate|up, down


def _fused(wl, layer, g):
    return np.concatenate([wl.weight(layer, i) for i in g], 0) if len(g) > 1 else wl.weight(layer, g[0])


def _check_matrix(wl, layer, g, batches, rng, nsample=48):
    w = _fused(wl, layer, g)
    n, k = w.shape
    name = "|".join(wl.linears[i].name for i in g)
    say(f"{wl.name} layer {layer} {name} {n}x{k} batches {batches}")
    pw = bg.quantize_groupwise(dev_bf16(w), 4, wl.symmetric, wl.group)
    rows = np.sort(rng.choice(n, nsample, replace=False))
    rows[0], rows[-1] = 0, n - 1  # first and last rows, plus the sample
    c_ref, s_ref, z_ref = oracle.quantize(w[rows], 4, wl.symmetric, wl.group)
    codes = host(pw.codes)
    assert_same_bits(codes[rows], c_ref, f"{name} codes (sampled rows)")
    assert_same_bits(host(pw.scales)[rows], s_ref, f"{name} scales (sampled rows)")
    if not wl.symmetric:
        assert_same_bits(host(pw.zeros)[rows], z_ref, f"{name} zeros (sampled rows)")
    for b in batches:
        x = wl.activation(k, b)
        y = host(bg.w4a16_gemv(dev_bf16(x), pw))
        assert np.all(np.isfinite(y))
        y_ref = oracle.w4a16_matmul(x, c_ref, s_ref, z_ref, rows.size, k, wl.symmetric, wl.group)
        assert_close(y[:, rows], y_ref, f"{name} y batch {b} (sampled rows)")
    del pw
    torch.cuda.empty_cache()


@pytest.mark.parametrize("gi", range(4))
def test_llama70b_decode_layer(gi):
    wl = WORKLOADS["llama70b_decode"]
    _check_matrix(wl, 0, GROUPS[gi], [1], np.random.default_rng(70 + gi))


@pytest.mark.parametrize("layer", [0, 31])
@pytest.mark.parametrize("gi", range(4))
def test_llama7b_decode_layer(layer, gi):
    wl = WORKLOADS["llama7b_decode"]
    _check_matrix(wl, layer, GROUPS[gi], [1, 4, 16], np.random.default_rng(7 + layer * 10 + gi))


def test_llama7b_outlier_channels_present():
    """The 7B stack's weights carry 1% of input channels x20 (checked on the
    data the GPU receives)."""
    wl = WORKLOADS["llama7b_decode"]
    w = wl.weight(0, 0, rows=np.arange(256)).astype(np.uint32) << 16
    col_abs = np.abs(w.view(np.float32)).mean(0)
    big = col_abs > 5 * np.median(col_abs)
    assert 35 <= big.sum() <= 45
