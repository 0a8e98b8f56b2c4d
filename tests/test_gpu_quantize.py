"""Bit-exact parity of quantize_groupwise / dequantize_groupwise with the oracle."""
import numpy as np
import pytest
import torch

import bit_gemv_amd as bg
import oracle
from gpu_helpers import assert_same_bits, dev, dev_bf16, host, say
from workloads import f32_to_bf16_bits, bf16_bits_to_f32

pytestmark = pytest.mark.gpu


def _run(w_bits, bits, sym, group, col_scale=None):
    n, k = w_bits.shape
    say(f"quantize n={n} k={k} bits={bits} sym={sym} group={group} cs={col_scale is not None}")
    cs_dev = None if col_scale is None else dev(col_scale.astype(np.float32))
    pw = bg.quantize_groupwise(dev_bf16(w_bits), bits, sym, group, cs_dev)
    c_ref, s_ref, z_ref = oracle.quantize(w_bits, bits, sym, group, col_scale)
    assert_same_bits(host(pw.codes), c_ref, "codes")
    assert_same_bits(host(pw.scales), s_ref, "scales")
    if not sym:
        assert_same_bits(host(pw.zeros), z_ref, "zeros")
    d_gpu = host(bg.dequantize_groupwise(pw))
    d_ref = oracle.dequantize(c_ref, s_ref, z_ref, n, k, bits, sym, group)
    assert_same_bits(d_gpu, d_ref, "dequantized")
    return pw


SHAPES = [(1, 128), (3, 384), (17, 2048 + 128), (64, 4096), (129, 11008)]


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("sym", [False, True])
@pytest.mark.parametrize("shape", SHAPES)
def test_random_normal(bits, sym, shape):
    rng = np.random.default_rng(hash((bits, sym, shape)) % 2 ** 32)
    w = f32_to_bf16_bits(rng.standard_normal(shape) * 0.02)
    _run(w, bits, sym, 128)


@pytest.mark.parametrize("bits,sym", [(4, False), (4, True), (8, True), (8, False)])
@pytest.mark.parametrize("group", ["k", 256, 1024])
def test_large_groups_and_per_channel(bits, sym, group):
    rng = np.random.default_rng(3)
    n, k = 37, 4096
    g = k if group == "k" else group
    w = f32_to_bf16_bits(rng.standard_normal((n, k)) * np.logspace(-3, 1, n)[:, None])
    _run(w, bits, sym, g)


# Groups of 128 M elements, M = 1..8, run on 16-lane teams with M loads per
# lane (and 4 / M groups per team for M <= 2); 115 groups leave the last
# block ragged. Column scales on per-channel rows (group == k).
@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("bits,sym", [(4, False), (4, True), (8, True), (8, False)])
def test_team_groups(m, bits, sym):
    group = 128 * m
    rng = np.random.default_rng(100 + 10 * m + bits + sym)
    n, k = 23, 5 * group
    w = f32_to_bf16_bits(rng.standard_normal((n, k)) * np.logspace(-2, 1, n)[:, None])
    _run(w, bits, sym, group)
    if bits == 8 and sym:
        w1 = f32_to_bf16_bits(rng.standard_normal((37, group)))
        _run(w1, bits, sym, group, np.exp(rng.uniform(-2, 2, group)).astype(np.float32))


# Groups above 1024 run one workgroup per group, four strides per lane held in
# registers at a time: 256 lanes (2048-element strides) up to 8192 elements,
# 1024 lanes (8192-element strides) above. A group of 2176 (a full and a
# partial stride), 3 or 4 full strides, 8320 (the first 1024-lane size),
# groups of 2 to 4 strides of 8192 (two groups per row, a partial last
# stride), then groups over two and three 32768-element chunks (re-read
# before their codes); per-channel groups with a column scale. (384 runs on
# the 16-lane teams above.)
@pytest.mark.parametrize("group,k", [(384, 1536), (2048 + 128, 4352), (6144, 6144), (8192, 8192),
                                     (8192 + 128, 8320), (3 * 8192 + 2048 + 128, 3 * 8192 + 2048 + 128),
                                     (16384, 32768), (28672, 28672), (32768 + 384, 32768 + 384),
                                     (2 * 32768 + 8192 + 128, 2 * 32768 + 8192 + 128)])
@pytest.mark.parametrize("bits,sym", [(8, True), (4, False)])
def test_large_group_strides(group, k, bits, sym):
    rng = np.random.default_rng(group + bits)
    n = 19
    w = f32_to_bf16_bits(rng.standard_normal((n, k)) * np.logspace(-2, 1, n)[:, None])
    cs = np.exp(rng.uniform(-2, 2, k)).astype(np.float32) if group == k else None
    _run(w, bits, sym, group, cs)


# Per-channel rows with column scales above 1024 channels: one row per block
# below k = 6144, two rows per block (sharing their column-scale loads) from
# there; an odd row count leaves the last block with one row.
@pytest.mark.parametrize("k", [1152, 4096 + 128, 6144, 8192])
@pytest.mark.parametrize("bits,sym", [(8, True), (8, False), (4, True), (4, False)])
def test_per_channel_col_scale_rows(k, bits, sym):
    rng = np.random.default_rng(k + 2 * bits + sym)
    n = 29
    w = f32_to_bf16_bits(rng.standard_normal((n, k)) * np.logspace(-2, 1, n)[:, None])
    cs = np.exp(rng.uniform(-2, 2, k)).astype(np.float32)
    _run(w, bits, sym, k, cs)


@pytest.mark.parametrize("bits,sym,group", [(8, True, "k"), (4, False, 128), (8, True, 128)])
def test_col_scale(bits, sym, group):
    rng = np.random.default_rng(4)
    n, k = 48, 2048
    w = f32_to_bf16_bits(rng.standard_normal((n, k)) * 0.02)
    cs = np.exp(rng.uniform(-3, 3, k)).astype(np.float32)
    _run(w, bits, sym, k if group == "k" else group, cs)


def _edge_matrix():
    """Degenerate and tie-heavy groups, 128 wide."""
    rows = []
    rows.append(np.zeros(128))                                   # all zero
    rows.append(np.full(128, 0.3))                               # constant
    rows.append(np.full(128, -1e20))                             # constant, large
    rows.append(np.linspace(0.5, 3.0, 128))                      # all positive (z < 0)
    rows.append(np.linspace(-3.0, -0.5, 128))                    # all negative (z > 15)
    r = np.zeros(128); r[0] = 7; r[1:9] = [2.5, 3.5, -2.5, 0.5, 1.5, -1.5, -0.5, 4.5]
    rows.append(r)                                               # sym ties (s = 1)
    r = np.zeros(128); r[0] = -5; r[1] = 10; r[2:8] = [2.5, -4.5, 3.5, -0.5, 6.5, 0.5]
    rows.append(r)                                               # asym ties (s = 1, z = 5)
    rng = np.random.default_rng(9)
    r = rng.uniform(-1, 1, 128); r[77] = 100.0
    rows.append(r)                                               # one outlier
    rows.append(rng.standard_normal(128) * 1e-38)                # subnormal-range values
    rows.append(rng.standard_normal(128) * 1e30)                 # huge but not constant
    rows.append(np.where(np.arange(128) % 2 == 0, 1e-30, -1e-30))
    rows.append(rng.standard_normal(128) * 1e-9)                 # range below the 1e-8 floor
    return f32_to_bf16_bits(np.stack(rows))


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("sym", [False, True])
def test_edge_groups(bits, sym):
    _run(_edge_matrix(), bits, sym, 128)


@pytest.mark.parametrize("sym", [False, True])
@pytest.mark.parametrize("shuffle", [False, True])
def test_every_finite_bf16_value(sym, shuffle):
    """All 65280 finite bf16 patterns (and some padding zeros), sorted so a
    group spans neighbouring values; optionally shuffled within rows."""
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    exp = (h >> 7) & 0xFF
    h = h[exp != 0xFF]
    v = bf16_bits_to_f32(h)
    h = h[np.argsort(v, kind="stable")]
    pad = (-h.size) % 256
    h = np.concatenate([h, np.zeros(pad, np.uint16)]).reshape(-1, 256)
    if shuffle:
        rng = np.random.default_rng(5)
        h = np.stack([rng.permutation(r) for r in h])
    _run(h, 4, sym, 128)
    _run(h, 8, sym, 128)


def _near_tie_groups(bits, sym, want, seed):
    """Groups (bf16, 128 wide) chosen from a large random pool because some
    element's IEEE fp32 quotient x / s lies closest to a rounding tie k + 1/2
    relative to its size: there a quotient one ulp off would change a code.
    s, z follow the definition in fp32 (numpy division is IEEE)."""
    rng = np.random.default_rng(seed)
    pool = 1 << 16
    # magnitudes from 2^-20 to 2^20 and shifted ranges, so that s, z and the
    # quotients spread over many binades (asymmetric groups away from zero)
    scale = np.exp2(rng.uniform(-20, 20, (pool, 1)))
    shift = rng.uniform(-3, 3, (pool, 1)) * (0 if sym else 1)
    w = f32_to_bf16_bits((rng.standard_normal((pool, 128)) + shift) * scale)
    x = bf16_bits_to_f32(w).astype(np.float32)
    if sym:
        qmax = np.float32((1 << (bits - 1)) - 1)
        s = np.maximum(np.abs(x).max(axis=1, keepdims=True), np.float32(1e-8)) / qmax
    else:
        levels = np.float32((1 << bits) - 1)
        mn, mx = x.min(axis=1, keepdims=True), x.max(axis=1, keepdims=True)
        s = np.maximum(mx - mn, np.float32(1e-8)) / levels
    q = (x / s.astype(np.float32)).astype(np.float32)
    d = np.abs(np.abs(q - np.floor(q)) - np.float32(0.5))
    ulps = d / np.spacing(np.abs(q).astype(np.float32))
    exact = (d == 0).any(axis=1)
    near = np.where(d == 0, np.inf, ulps).min(axis=1)  # closest miss, in ulps
    order = np.argsort(near)
    best = np.concatenate([order[: want - want // 4], np.flatnonzero(exact)[: want // 4]])
    best = np.concatenate([best, order[want - want // 4: want - want // 4 + (want - best.size)]])
    return w[best]


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("sym", [False, True])
def test_quotients_next_to_rounding_ties(bits, sym):
    """Codes where x / s sits within a few ulps of k + 1/2 must follow the
    IEEE quotient exactly (the kernel divides with FMA corrections)."""
    w = _near_tie_groups(bits, sym, 2048, seed=bits * 2 + sym)
    _run(w.reshape(-1, 8 * 128), bits, sym, 128)


def test_empty_matrix_is_noop():
    w = torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda")
    pw = bg.quantize_groupwise(w, 4, True, 128)
    assert pw.codes.shape == (0, 128)


def test_outputs_untouched_on_rejected_call():
    w = torch.zeros((4, 256), dtype=torch.bfloat16, device="cuda")
    pw = bg.quantize_groupwise(w, 4, False, 128)
    before = pw.codes.clone()
    with pytest.raises(bg.LibquantError):
        bg._call("quantize_groupwise", bg._ptr(w), 4, 256, 4, 1, 128, None, bg._ptr(pw.codes),
                 bg._ptr(pw.scales), bg._ptr(pw.zeros), bg._stream())
    torch.cuda.synchronize()
    assert torch.equal(before, pw.codes)
