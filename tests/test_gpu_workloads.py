"""Parity at the workloads' full sizes, in the launch configurations the
benchmark times (fused q|k|v and gate|up matrices; the 70B stack at batch
1, 4 and 16 in INT4, INT8 and MXFP4, the 7B stack in INT4 at batch 1, 4
and 16), on seeded samples of rows the oracle computes one by one."""
import numpy as np
import pytest
import torch

import bit_gemv_amd as bg
import oracle
from gpu_helpers import assert_close, assert_same_bits, dev_bf16, host, say
from workloads import WORKLOADS, tp8_share_weights

pytestmark = pytest.mark.gpu

GROUPS = [[0, 1, 2], [3], [4, 5], [6]]  # q|k|v, o, gate|up, down


def _fused(wl, layer, g):
    return np.concatenate([wl.weight(layer, i) for i in g], 0) if len(g) > 1 else wl.weight(layer, g[0])


def _rows_of(t, rows):
    return host(t[torch.from_numpy(rows).cuda()])


def _check_matrix(wl, layer, g, batches, rng, nsample=48, formats=("int4",)):
    w = _fused(wl, layer, g)
    n, k = w.shape
    name = "|".join(wl.linears[i].name for i in g)
    rows = np.sort(rng.choice(n, nsample, replace=False))
    rows[0], rows[-1] = 0, n - 1  # first and last rows, plus the sample
    wd = dev_bf16(w)
    xs = {b: wl.activation(k, b) for b in batches}
    for fmt in formats:
        say(f"{wl.name} layer {layer} {name} {n}x{k} {fmt} batches {batches}")
        if fmt == "mxfp4":
            mw = bg.mxfp4_quantize(wd)
            c_ref, s_ref = oracle.mx_quantize(w[rows])
            assert_same_bits(_rows_of(mw.codes, rows), c_ref, f"{name} mxfp4 codes (sampled rows)")
            assert_same_bits(_rows_of(mw.scales, rows), s_ref, f"{name} mxfp4 scales (sampled rows)")
            for b in batches:
                y = host(bg.mxfp4_gemv(dev_bf16(xs[b]), mw))
                assert np.all(np.isfinite(y))
                assert_close(y[:, rows], oracle.mx_matmul(xs[b], c_ref, s_ref, rows.size, k),
                             f"{name} mxfp4 y batch {b} (sampled rows)")
            del mw
        else:
            bits = 4 if fmt == "int4" else 8
            pw = bg.quantize_groupwise(wd, bits, wl.symmetric, wl.group)
            c_ref, s_ref, z_ref = oracle.quantize(w[rows], bits, wl.symmetric, wl.group)
            assert_same_bits(_rows_of(pw.codes, rows), c_ref, f"{name} {fmt} codes (sampled rows)")
            assert_same_bits(_rows_of(pw.scales, rows), s_ref, f"{name} {fmt} scales (sampled rows)")
            if not wl.symmetric:
                assert_same_bits(_rows_of(pw.zeros, rows), z_ref, f"{name} {fmt} zeros (sampled rows)")
            gemv = bg.w4a16_gemv if bits == 4 else bg.w8a16_gemv
            matmul = oracle.w4a16_matmul if bits == 4 else oracle.w8a16_matmul
            for b in batches:
                y = host(gemv(dev_bf16(xs[b]), pw))
                assert np.all(np.isfinite(y))
                y_ref = matmul(xs[b], c_ref, s_ref, z_ref, rows.size, k, wl.symmetric, wl.group)
                assert_close(y[:, rows], y_ref, f"{name} {fmt} y batch {b} (sampled rows)")
            del pw
        torch.cuda.empty_cache()
    del wd
    torch.cuda.empty_cache()


@pytest.mark.parametrize("gi", range(4))
def test_llama70b_decode_layer(gi):
    """Each fused 70B matrix in the three weight formats the benchmark's
    decode sweeps time (INT4 and INT8 asymmetric G = 128, MXFP4), at batch
    1, 4 and 16 (the VALU, split-run shared-stage and single-run kernels)."""
    wl = WORKLOADS["llama70b_decode"]
    _check_matrix(wl, 0, GROUPS[gi], [1, 4, 16], np.random.default_rng(70 + gi),
                  formats=("int4", "int8", "mxfp4"))


@pytest.mark.parametrize("j", range(4))
def test_llama70b_tp8_share(j):
    """One GPU's share of an 8-way tensor-parallel 70B layer (the shapes the
    benchmark's tp8_share_decode row times): codes of sampled rows bit-exact
    and batch-1 outputs of those rows against the oracle."""
    wl = WORKLOADS["llama70b_decode"]
    w = tp8_share_weights(wl, 0)[j]
    n, k = w.shape
    say(f"tp8 share {n}x{k}")
    pw = bg.quantize_groupwise(dev_bf16(w), 4, wl.symmetric, wl.group)
    rows = np.sort(np.random.default_rng(80 + j).choice(n, 48, replace=False))
    rows[0], rows[-1] = 0, n - 1
    c_ref, s_ref, z_ref = oracle.quantize(w[rows], 4, wl.symmetric, wl.group)
    assert_same_bits(_rows_of(pw.codes, rows), c_ref, "codes (sampled rows)")
    assert_same_bits(_rows_of(pw.scales, rows), s_ref, "scales (sampled rows)")
    assert_same_bits(_rows_of(pw.zeros, rows), z_ref, "zeros (sampled rows)")
    x = wl.activation(k, 1)
    y = host(bg.w4a16_gemv(dev_bf16(x), pw))
    assert_close(y[:, rows], oracle.w4a16_matmul(x, c_ref, s_ref, z_ref, rows.size, k, wl.symmetric, wl.group),
                 "y batch 1 (sampled rows)")


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
