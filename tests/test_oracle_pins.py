"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these retype the oracle's formulas: they check printed values,
brute-force searches, bounds, invariants and library routines, so that a
dropped term, a wrong sign or index, or a transposed operand in ``oracle.c``
fails at least one of them.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

f32 = np.float32


@pytest.fixture(scope="module")
def golden(golden_dir):
    with open(os.path.join(golden_dir, "worked_int4_example.json")) as f:
        worked = json.load(f)
    with open(os.path.join(golden_dir, "printed_values.json")) as f:
        printed = json.load(f)
    return worked, printed


def _unpack4(codes, k):
    lo = (codes & 0xF).astype(np.int32)
    hi = (codes >> 4).astype(np.int32)
    out = np.empty((codes.shape[0], k), np.int32)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


def _signed_codes(codes, k, bits, symmetric):
    if bits == 4:
        u = _unpack4(codes, k)
        return u - 8 if symmetric else u
    return codes.view(np.int8).astype(np.int32) if symmetric else codes.astype(np.int32)


# --------------------------------------------------------------------------
# Worked example, "3.6 Quantization" page: 8 weights to INT4, both modes.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("mode", ["symmetric", "asymmetric"])
def test_worked_int4_example(golden, mode):
    worked, _ = golden
    ref = worked[mode]
    w = np.array(worked["w"], f32)[None, :]
    sym = mode == "symmetric"
    codes, s, z = oracle.quantize(w, 4, sym, 8)
    q = _signed_codes(codes, 8, 4, sym)[0]
    assert q.tolist() == ref["q"]
    assert abs(float(s[0, 0]) - ref["s"]) < 1e-4
    if not sym:
        assert float(z[0, 0]) == ref["z"]
    w_hat = oracle.dequantize(codes, s, z, 1, 8, 4, sym, 8)[0]
    assert np.allclose(w_hat, ref["w_hat"], atol=5e-4)
    mse = float(np.mean((w_hat.astype(np.float64) - w[0]) ** 2))
    assert abs(mse - ref["mse"]) < 0.01e-3
    # the page's remark: asymmetric MSE is about 25% lower than symmetric
    if not sym:
        assert mse < worked["symmetric"]["mse"]


def test_int8_selftest(golden):
    _, p = golden
    t = p["int8_selftest"]
    w = np.array([[t["amax"], t["x"], 0, 0, 0, 0, 0, -0.3]], f32)
    codes, s, _ = oracle.quantize(w, 8, True, 8)
    assert s[0, 0] == f32(t["s"])
    assert int(codes.view(np.int8)[0, 1]) == t["q"]
    assert int(codes.view(np.int8)[0, 0]) == 127


def test_outlier_collapses_normals_to_zero():
    """"Intuition" section of the "3.6 Quantization" page: one 100 among values
    of size ~1 makes the 4-bit step about 100/7 and every normal value rounds
    to 0."""
    rng = np.random.default_rng(7)
    g = rng.uniform(-1, 1, 128).astype(f32)
    g[37] = 100.0
    codes, s, _ = oracle.quantize(g[None, :], 4, True, 128)
    q = _signed_codes(codes, 128, 4, True)[0]
    assert abs(float(s[0, 0]) - 100 / 7) < 1e-5
    assert q[37] == 7
    assert np.count_nonzero(np.delete(q, 37)) == 0


# --------------------------------------------------------------------------
# Rounding rule: half to even, applied to x/s before adding z.
# --------------------------------------------------------------------------
def test_symmetric_ties_round_half_even():
    # amax 7 -> s = 7/7 = 1 exactly, so x/s = x and ties are exact
    w = np.array([[7.0, 2.5, 3.5, -2.5, 0.5, 1.5, -1.5, -0.5]], f32)
    codes, s, _ = oracle.quantize(w, 4, True, 8)
    assert s[0, 0] == 1.0
    assert _signed_codes(codes, 8, 4, True)[0].tolist() == [7, 2, 4, -2, 0, 2, -2, 0]


def test_asymmetric_rounds_before_adding_zero_point():
    # min -5, max 10 -> s = 1, z = 5 (odd): round(2.5) + 5 = 7, while round(7.5) = 8
    w = np.array([[-5.0, 10.0, 2.5, -4.5, 3.5, 0.0, -0.5, 6.5]], f32)
    codes, s, z = oracle.quantize(w, 4, False, 8)
    assert s[0, 0] == 1.0 and z[0, 0] == 5.0
    assert _unpack4(codes, 8)[0].tolist() == [0, 15, 7, 1, 9, 5, 5, 11]


def test_zero_point_negative_zero_is_canonical():
    # min 0 -> -min/s = -0.0 -> z must be +0.0
    w = np.array([[0.0, 1.0, 0.5, 0.25, 0.75, 0.1, 0.2, 0.3]], f32)
    _, _, z = oracle.quantize(w, 4, False, 8)
    assert z[0, 0] == 0.0 and not np.signbit(z[0, 0])


# --------------------------------------------------------------------------
# Brute force: each code is the nearest reconstruction level, exactly.
# --------------------------------------------------------------------------
def _brute_force_check(x, s, z, q, bits, symmetric):
    """For one group: q must minimise |x - s (c - z)| over the code range,
    in exact rational arithmetic; exact ties must land on the even (c - z)."""
    if symmetric:
        qmax = 2 ** (bits - 1) - 1
        cand = range(-qmax, qmax + 1)
        zf = Fraction(0)
    else:
        cand = range(0, 2 ** bits)
        zf = Fraction(float(z))
    sf = Fraction(float(s))
    checked = 0
    for xi, qi in zip(x, q):
        xf = Fraction(float(xi))
        ratio = xf / sf
        frac = ratio - (ratio.numerator // ratio.denominator)
        if abs(frac - Fraction(1, 2)) < Fraction(1, 10 ** 5):
            continue  # within fp32 rounding of a half-way point: x/s decides
        d = [abs(xf - sf * (c - zf)) for c in cand]
        best = min(d)
        winners = [c for c, dv in zip(cand, d) if dv == best]
        assert int(qi) in winners, (xi, s, z, qi, winners)
        checked += 1
    return checked


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("symmetric", [True, False])
def test_brute_force_nearest_code(bits, symmetric):
    rng = np.random.default_rng(100 + bits + 10 * symmetric)
    n, g = 6, 16
    w = rng.standard_normal((n, 4 * g)).astype(f32)
    w[1] = np.abs(w[1]) + 0.5            # group not straddling zero (z outside code range)
    w[2] *= 1e-3
    w[3, :g] = 0.25                      # constant group (range floored)
    w[4, :g] = 0.0                       # all-zero group
    codes, s, z = oracle.quantize(w, bits, symmetric, g)
    q = _signed_codes(codes, w.shape[1], bits, symmetric)
    checked = 0
    for r in range(n):
        for gi in range(4):
            sl = slice(gi * g, (gi + 1) * g)
            checked += _brute_force_check(w[r, sl], s[r, gi], None if symmetric else z[r, gi],
                                          q[r, sl], bits, symmetric)
    assert checked > n * 4 * g * 0.9


# --------------------------------------------------------------------------
# Properties of s and z stated on the pages.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("symmetric", [True, False])
def test_error_at_most_half_step(bits, symmetric):
    """"Symmetric and asymmetric quantization", "3.6 Quantization": without
    clipping every element's rounding error is at most s/2."""
    rng = np.random.default_rng(5 + bits)
    w = np.concatenate([rng.standard_normal((8, 512)), rng.uniform(-3, 5, (8, 512)),
                        rng.standard_t(2, (8, 512))]).astype(f32)
    codes, s, z = oracle.quantize(w, bits, symmetric, 128)
    w_hat = oracle.dequantize(codes, s, z, w.shape[0], w.shape[1], bits, symmetric, 128)
    half = np.repeat(s, 128, axis=1).astype(np.float64) / 2
    err = np.abs(w_hat.astype(np.float64) - w)
    assert np.all(err <= half * (1 + 1e-5) + 1e-12)


@pytest.mark.parametrize("bits", [4, 8])
def test_asymmetric_grid_spans_min_to_max(bits):
    """The asymmetric grid covers [min x, max x]: 2^b - 1 steps of s span the
    range, and the level of code 0 sits within s/2 of min x."""
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((16, 256)) * 0.02 + 0.003).astype(f32)
    codes, s, z = oracle.quantize(w, bits, False, 128)
    g = w.reshape(16, 2, 128)
    rng_ = g.max(-1).astype(np.float64) - g.min(-1)
    assert np.allclose(s * (2 ** bits - 1), rng_, rtol=1e-6)
    assert np.all(z == np.round(z))
    lvl0 = -z.astype(np.float64) * s
    assert np.all(np.abs(lvl0 - g.min(-1)) <= s / 2 * (1 + 1e-5))


def test_symmetric_grid_top_level_is_absmax():
    rng = np.random.default_rng(12)
    w = rng.standard_normal((8, 384)).astype(f32)
    codes, s, _ = oracle.quantize(w, 4, True, 128)
    amax = np.abs(w.reshape(8, 3, 128)).max(-1)
    assert np.allclose(s * 7, amax, rtol=1e-6)
    q = _signed_codes(codes, 384, 4, True).reshape(8, 3, 128)
    assert q.max() <= 7 and q.min() >= -7
    # the element holding max|x| maps to +-qmax
    idx = np.abs(w.reshape(8, 3, 128)).argmax(-1)
    top = np.take_along_axis(np.abs(q), idx[..., None], -1)[..., 0]
    assert np.all(top == 7)


def test_group_k_is_per_channel_and_single_row_is_per_tensor():
    """Granularity special cases: with group = k there is one scale per output
    row; a matrix flattened to one row with group = its size has one scale."""
    rng = np.random.default_rng(13)
    w = (rng.standard_normal((4, 256)) * np.array([[0.01], [0.1], [1], [10]])).astype(f32)
    _, s_row, _ = oracle.quantize(w, 8, True, 256)
    assert s_row.shape == (4, 1)
    assert np.allclose(s_row[:, 0] * 127, np.abs(w).max(1), rtol=1e-6)
    _, s_t, _ = oracle.quantize(w.reshape(1, -1), 8, True, w.size)
    assert s_t.shape == (1, 1) and np.isclose(s_t[0, 0] * 127, np.abs(w).max(), rtol=1e-6)


def test_toy_granularity_ratio(golden):
    """Code block of "3.6 Quantization": on rows scaled by logspace(-2, 0),
    per-group-128 INT4 error is about a third of per-tensor INT4 error."""
    _, p = golden
    rng = np.random.default_rng(0)
    W = (rng.standard_normal((256, 1024)).astype(f32)
         * np.logspace(-2, 0, 256, dtype=f32)[:, None]).astype(f32)

    def rel_err(A, G):
        c, s, z = oracle.quantize(A, 4, True, G)
        d = oracle.dequantize(c, s, z, A.shape[0], A.shape[1], 4, True, G).reshape(W.shape)
        return np.linalg.norm(W - d) / np.linalg.norm(W)

    e_tensor = rel_err(W.reshape(1, -1), W.size)
    e_channel = rel_err(W, 1024)
    e_group = rel_err(W, 128)
    ratio = e_tensor / e_group
    assert e_group < e_channel < e_tensor
    assert 2.0 <= ratio <= 4.5, ratio  # printed: about 3
    assert abs(ratio - p["toy_ratios"]["per_tensor_over_per_group"]) < 1.5


# --------------------------------------------------------------------------
# Effective bits and byte accounting.
# --------------------------------------------------------------------------
def test_effective_bits_printed_values(golden):
    _, p = golden
    for c in p["effective_bits"]["cases"]:
        assert oracle.effective_bits(c["bits"], c["scale_bits"], c["zero_bits"], c["group"]) == c["value"]


def test_model_size_table(golden):
    _, p = golden
    t = p["model_sizes_70b"]
    for c in t["cases"]:
        eb = oracle.effective_bits(c["bits"], c["scale_bits"], c["zero_bits"], c["group"])
        assert round(t["params"] * eb / 8 / 1e9) == c["gb"]


def test_packed_bytes_match_effective_bits():
    # fp32 scale (+ fp32 zero) per 128 weights: 4 + 32/128 = 4.25, 4 + 64/128 = 4.5
    n, k = 4096, 4096
    assert oracle.packed_bytes(n, k, 4, True, 128) * 8 / (n * k) == oracle.effective_bits(4, 32, 0, 128) == 4.25
    assert oracle.packed_bytes(n, k, 4, False, 128) * 8 / (n * k) == oracle.effective_bits(4, 32, 32, 128) == 4.5
    codes, s, z = oracle.quantize(np.zeros((4, 256), f32), 4, False, 128)
    assert codes.nbytes + s.nbytes + z.nbytes == oracle.packed_bytes(4, 256, 4, False, 128)


# --------------------------------------------------------------------------
# W4A16 matmul: y = x W_hat^T.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("symmetric", [True, False])
def test_w4a16_matmul_is_x_times_dequantized_transpose(symmetric):
    from workloads import f32_to_bf16_bits, bf16_bits_to_f32
    rng = np.random.default_rng(21)
    n, k, m = 24, 384, 3
    w = f32_to_bf16_bits(rng.standard_normal((n, k)) * 0.02)
    x = f32_to_bf16_bits(rng.standard_normal((m, k)))
    codes, s, z = oracle.quantize(w, 4, symmetric, 128)
    y = oracle.w4a16_matmul(x, codes, s, z, n, k, symmetric, 128)
    w_hat = oracle.dequantize(codes, s, z, n, k, 4, symmetric, 128).astype(np.float64)
    ref = bf16_bits_to_f32(x).astype(np.float64) @ w_hat.T
    assert y.shape == (m, n)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)
    # and close to the unquantized product (INT4 error, not a layout slip)
    full = bf16_bits_to_f32(x).astype(np.float64) @ bf16_bits_to_f32(w).astype(np.float64).T
    rel = np.linalg.norm(y - full) / np.linalg.norm(full)
    assert rel < 0.2


def test_w4a16_matmul_closed_form():
    """One-hot activations pick single dequantized weights; a constant
    activation sums a row."""
    rng = np.random.default_rng(22)
    n, k = 5, 256
    w = rng.standard_normal((n, k)).astype(f32)
    codes, s, z = oracle.quantize(w, 4, False, 128)
    w_hat = oracle.dequantize(codes, s, z, n, k, 4, False, 128)
    x = np.zeros((2, k), np.uint16)
    x[0, 77] = 0x3F80  # bf16 1.0
    x[1, :] = 0x4000   # bf16 2.0
    y = oracle.w4a16_matmul(x, codes, s, z, n, k, False, 128)
    assert np.array_equal(y[0], w_hat[:, 77].astype(np.float64))
    assert np.allclose(y[1], 2 * w_hat.astype(np.float64).sum(1), rtol=1e-12)


@pytest.mark.parametrize("symmetric", [False, True])
def test_w8a16_matmul_is_x_times_dequantized_transpose(symmetric):
    from workloads import f32_to_bf16_bits, bf16_bits_to_f32
    rng = np.random.default_rng(23)
    n, k, m = 19, 512, 4
    w = f32_to_bf16_bits(rng.standard_normal((n, k)) * 0.02)
    x = f32_to_bf16_bits(rng.standard_normal((m, k)))
    codes, s, z = oracle.quantize(w, 8, symmetric, 128)
    assert codes.size == n * k  # one byte per weight
    y = oracle.w8a16_matmul(x, codes, s, z, n, k, symmetric, 128)
    w_hat = oracle.dequantize(codes, s, z, n, k, 8, symmetric, 128).astype(np.float64)
    ref = bf16_bits_to_f32(x).astype(np.float64) @ w_hat.T
    assert y.shape == (m, n)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)
    # INT8 is far closer to the unquantized product than INT4 would be
    full = bf16_bits_to_f32(x).astype(np.float64) @ bf16_bits_to_f32(w).astype(np.float64).T
    rel = np.linalg.norm(y - full) / np.linalg.norm(full)
    assert rel < 0.01


@pytest.mark.parametrize("symmetric", [False, True])
def test_w8a16_matmul_hand_built_codes(symmetric):
    """Codes, scales and zero-points built by hand (not by the quantizer):
    signed two's-complement bytes for symmetric, unsigned bytes with a
    zero-point for asymmetric. Power-of-two scales and small-integer
    activations make every product and sum exact, so the result must equal
    sum_j x_j (q_j - z) s bit for bit, group by group."""
    rng = np.random.default_rng(24)
    n, k, g = 6, 384, 128
    ng = k // g
    if symmetric:
        q = rng.integers(-128, 128, (n, k))
        codes = (q & 0xFF).astype(np.uint8)
        z = np.zeros((n, ng), f32)
    else:
        q = rng.integers(0, 256, (n, k))
        codes = q.astype(np.uint8)
        z = rng.integers(0, 256, (n, ng)).astype(f32)
    s = (2.0 ** rng.integers(-12, -2, (n, ng))).astype(f32)
    xi = rng.integers(-8, 9, (2, k))
    x = (np.float32(1.0) * xi).astype(f32).view(np.uint32)
    x = (x >> 16).astype(np.uint16)  # small integers are exact in bf16
    y = oracle.w8a16_matmul(x, codes, s, None if symmetric else z, n, k, symmetric, g)
    expect = np.zeros((2, n))
    for i in range(2):
        for r in range(n):
            for gi in range(ng):
                sl = slice(gi * g, (gi + 1) * g)
                expect[i, r] += float(s[r, gi]) * float(np.dot(xi[i, sl], q[r, sl] - z[r, gi]))
    assert np.array_equal(y, expect)


# --------------------------------------------------------------------------
# SmoothQuant.
# --------------------------------------------------------------------------
def test_smoothquant_selftest(golden):
    _, p = golden
    t = p["smoothquant_selftest"]
    s = oracle.smooth_scale_from_absmax([t["ax"]], [t["aw"]], t["alpha"])
    assert s[0] == f32(t["s"])
    assert f32(t["ax"]) / s[0] == f32(t["new_max_x"])
    assert f32(t["aw"]) * s[0] == f32(t["new_max_w"])


@pytest.mark.parametrize("alpha", [0.5, 0.3, 0.8])
def test_smoothing_equalises_channel_maxima(alpha):
    """SmoothQuant section: after smoothing, max|X_hat_j| = ax^(1-a) aw^(1-a)
    and max|W_hat_j| = ax^a aw^a; both are sqrt(ax aw) at alpha 0.5."""
    rng = np.random.default_rng(31)
    ax = np.exp(rng.uniform(-2, 5, 200)).astype(f32)
    aw = np.exp(rng.uniform(-6, 0, 200)).astype(f32)
    s = oracle.smooth_scale_from_absmax(ax, aw, alpha).astype(np.float64)
    axd, awd = ax.astype(np.float64), aw.astype(np.float64)
    assert np.allclose(axd / s, axd ** (1 - alpha) * awd ** (1 - alpha), rtol=1e-5)
    assert np.allclose(awd * s, axd ** alpha * awd ** alpha, rtol=1e-5)
    if alpha == 0.5:
        assert np.allclose(axd / s, np.sqrt(axd * awd), rtol=3e-7)


def test_smooth_scale_reads_channel_maxima_on_the_right_axes():
    """ax is a max over tokens (rows of X[t][k]); aw a max over output rows of
    W[n][k] (the weight row that multiplies input channel j in Y = X W)."""
    from workloads import f32_to_bf16_bits
    x = np.zeros((3, 4), f32)
    x[2, 1] = -16.0   # channel 1 max over tokens
    x[0, 3] = 4.0
    w = np.zeros((5, 4), f32)
    w[4, 1] = 0.25    # input channel 1 max over output rows
    w[1, 3] = 1.0
    s = oracle.smooth_scale(f32_to_bf16_bits(x), f32_to_bf16_bits(w), 0.5)
    assert s[1] == f32(8.0)          # sqrt(16) / sqrt(0.25)
    assert s[3] == f32(2.0)          # sqrt(4) / sqrt(1)
    assert s[0] == f32(1.0)          # both floored at 1e-8


def _page_toy_smoothquant(seed):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((64, 1024)).astype(f32)
    X[:, :8] *= 50
    Wp = (rng.standard_normal((1024, 1024)) / 32).astype(f32)  # page layout W[C_in][C_out]
    W = np.ascontiguousarray(Wp.T)                                # our W[n][k]
    return X, W


def test_smoothing_is_exact_and_reduces_w8a8_error(golden):
    """Code block of "3.6 Quantization": (X diag(s)^-1)(diag(s) W) == X W, and
    smoothing lowers the W8A8 output error about 4x."""
    _, p = golden
    X, W = _page_toy_smoothquant(0)
    Y = X.astype(np.float64) @ W.astype(np.float64).T
    ax = np.abs(X).max(0)
    aw = np.abs(W).max(0)
    s = oracle.smooth_scale_from_absmax(ax, aw, 0.5)
    # exact identity in fp64 with the oracle's s
    Xs = X.astype(np.float64) / s
    Ws = W.astype(np.float64) * s
    assert np.allclose(Xs @ Ws.T, Y, rtol=1e-10, atol=1e-10)

    def w8a8(smooth):
        qx, sx = oracle.quant_per_token_int8(X, smooth)
        qw, sw, _ = oracle.quantize(W, 8, True, W.shape[1], col_scale=smooth)
        acc, y = oracle.w8a8_gemm(qx, sx, qw.view(np.int8), sw[:, 0])
        return y

    e_plain = np.linalg.norm(Y - w8a8(None)) / np.linalg.norm(Y)
    e_smooth = np.linalg.norm(Y - w8a8(s)) / np.linalg.norm(Y)
    ratio = e_plain / e_smooth
    assert 2.5 <= ratio <= 8.0, ratio  # printed: about 4x
    assert e_smooth < 0.02


def test_per_token_int8_brute_force():
    rng = np.random.default_rng(41)
    x = (rng.standard_normal((4, 32)) * np.array([[1], [30], [1e-3], [5]])).astype(f32)
    sm = np.exp(rng.uniform(-1, 1, 32)).astype(f32)
    qx, sx = oracle.quant_per_token_int8(x, sm)
    xs = x / sm  # fp32 division, as the smoothing step
    assert np.allclose(sx * 127, np.abs(xs).max(1), rtol=1e-6)
    for t in range(4):
        _brute_force_check(xs[t], sx[t], None, qx[t].astype(np.int32), 8, True)


def test_w8a8_accumulators_match_int64_matmul():
    rng = np.random.default_rng(51)
    m, n, k = 7, 9, 1024
    qx = rng.integers(-127, 128, (m, k), dtype=np.int8)
    qw = rng.integers(-127, 128, (n, k), dtype=np.int8)
    qx[0, :] = 127
    qw[0, :] = 127            # largest magnitude sum: k * 127^2 fits int32
    qw[1, :] = -127
    sx = rng.uniform(0.01, 1, m).astype(f32)
    sw = rng.uniform(0.01, 1, n).astype(f32)
    acc, y = oracle.w8a8_gemm(qx, sx, qw, sw)
    ref = qx.astype(np.int64) @ qw.astype(np.int64).T
    assert np.array_equal(acc.astype(np.int64), ref)
    assert np.allclose(y, ref * sx[:, None].astype(np.float64) * sw[None, :].astype(np.float64),
                       rtol=1e-15)


def test_int32_accumulator_bound_for_largest_k():
    # K * 127^2 < 2^31 for the largest input dimension used (28672)
    assert 28672 * 127 * 127 < 2 ** 31


def test_invalid_arguments_rejected():
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros((2, 100), f32), 4, True, 128)


# --------------------------------------------------------------------------
# AWQ activation-aware scaling ("3.6 Quantization", AWQ section).
# --------------------------------------------------------------------------
def _bf16_rne_np(a):
    from workloads import f32_to_bf16_bits, bf16_bits_to_f32
    return bf16_bits_to_f32(f32_to_bf16_bits(np.asarray(a, np.float32)))


def _awq_case(seed, t=24, n=40, k=384, outliers=(7, 200), mult=30.0):
    from workloads import f32_to_bf16_bits
    rng = np.random.default_rng(seed)
    xf = rng.standard_normal((t, k)).astype(f32)
    xf[:, list(outliers)] *= f32(mult)
    x = f32_to_bf16_bits(xf)
    w = f32_to_bf16_bits(rng.standard_normal((n, k)) * 0.02)
    return x, w


def test_act_absmean_is_the_channel_mean_magnitude():
    from workloads import bf16_bits_to_f32
    x, _ = _awq_case(30)
    sx = oracle.act_absmean(x)
    ref = np.abs(bf16_bits_to_f32(x).astype(np.float64)).mean(axis=0)
    assert np.array_equal(sx, ref.astype(f32))


def test_awq_scale_grid_ends():
    """alpha = 0 gives s = 1 (plain RTN); alpha = 1 gives s = s_X; a zero
    channel is floored at 1e-8 first."""
    sx = np.array([0.5, 2.0, 0.0, 37.25], f32)
    assert np.array_equal(oracle.awq_scale(sx, 0, 20), np.ones(4, f32))
    assert np.array_equal(oracle.awq_scale(sx, 20, 20), np.array([0.5, 2.0, 1e-8, 37.25], f32))
    half = oracle.awq_scale(sx, 10, 20)
    assert np.allclose(half, np.sqrt(np.maximum(sx, 1e-8)), rtol=1e-6)


@pytest.mark.parametrize("symmetric", [False, True])
def test_awq_loss_recomputed_in_numpy(symmetric):
    """The loss from its definition: quantize W diag(s) (pinned quantizer),
    dequantize, X / s rounded to bf16, fp64 products."""
    from workloads import bf16_bits_to_f32
    x, w = _awq_case(31)
    t, k = x.shape
    n = w.shape[0]
    rng = np.random.default_rng(5)
    s = np.exp(rng.uniform(-1.0, 1.5, k)).astype(f32)
    got = oracle.awq_loss(x, w, s, 4, symmetric, 128)
    codes, sc, z = oracle.quantize(w, 4, symmetric, 128, col_scale=s)
    w_hat = oracle.dequantize(codes, sc, z, n, k, 4, symmetric, 128).astype(np.float64)
    xf = bf16_bits_to_f32(x)
    xs = _bf16_rne_np(xf / s).astype(np.float64)
    y_ref = xf.astype(np.float64) @ bf16_bits_to_f32(w).astype(np.float64).T
    ref = float(((y_ref - xs @ w_hat.T) ** 2).sum())
    assert got == pytest.approx(ref, rel=1e-12)


def test_awq_alpha_zero_is_plain_rtn():
    """At alpha = 0 the search evaluates plain group-wise RTN."""
    from workloads import bf16_bits_to_f32
    x, w = _awq_case(32)
    t, k = x.shape
    n = w.shape[0]
    sx, losses, best, s_best = oracle.awq_search(x, w, 4, False, 128, 20)
    codes, sc, z = oracle.quantize(w, 4, False, 128)
    w_hat = oracle.dequantize(codes, sc, z, n, k, 4, False, 128).astype(np.float64)
    xf = bf16_bits_to_f32(x).astype(np.float64)
    rtn = float(((xf @ bf16_bits_to_f32(w).astype(np.float64).T - xf @ w_hat.T) ** 2).sum())
    assert losses[0] == pytest.approx(rtn, rel=1e-12)
    assert losses.shape == (21,)
    assert best == int(np.argmin(losses))
    assert np.array_equal(s_best, oracle.awq_scale(sx, best, 20))


def test_awq_search_protects_outlier_channels():
    """The AWQ section's claim: with a few activation channels far larger
    than the rest, scaling them before RTN lowers the output error, so the
    search lands on alpha > 0 and beats plain RTN clearly."""
    x, w = _awq_case(33, t=32, n=64, k=512, outliers=(3, 77, 300, 411), mult=40.0)
    _, losses, best, _ = oracle.awq_search(x, w, 4, False, 128, 20)
    assert best > 0
    assert losses[best] < 0.8 * losses[0]


def test_awq_scaling_shrinks_a_channels_error_about_1_over_s():
    """The AWQ section: multiplying one weight channel by s leaves the group
    range (set by the other weights) unchanged, so its rounding error after
    dividing by s falls by about 1/s. Over many groups, channel 5 scaled by
    4 has a mean absolute error near a quarter of the unscaled one."""
    rng = np.random.default_rng(34)
    n, k = 2000, 128
    w = rng.uniform(-1.0, 1.0, (n, k)).astype(f32)
    w[:, 0], w[:, 1] = 1.0, -1.0          # every group's range is [-1, 1]
    w[:, 5] *= f32(0.2)                   # scaled by 4 it stays inside the range
    s = np.ones(k, f32)
    s[5] = 4.0
    def err(cs):
        codes, sc, z = oracle.quantize(w, 4, False, 128, col_scale=cs)
        w_hat = oracle.dequantize(codes, sc, z, n, k, 4, False, 128)
        return np.abs(w_hat[:, 5] / cs[5] - w[:, 5]).mean()
    e1, e4 = err(np.ones(k, f32)), err(s)
    assert 0.18 < e4 / e1 < 0.32


# --------------------------------------------------------------------------
# MXFP4 (number-format table of "3.6 Quantization"; compendium MX formats).
# --------------------------------------------------------------------------
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _mx_block_rows(vals):
    """bf16 bits of a [rows][32k] float array (values must be exact in bf16)."""
    from workloads import f32_to_bf16_bits, bf16_bits_to_f32
    a = np.asarray(vals, np.float32)
    h = f32_to_bf16_bits(a)
    assert np.array_equal(bf16_bits_to_f32(h), a)
    return h


def _nibbles(codes, k):
    lo = (codes & 0xF).astype(np.int32)
    hi = (codes >> 4).astype(np.int32)
    out = np.empty((codes.shape[0], k), np.int32)
    out[:, 0::2], out[:, 1::2] = lo, hi
    return out


def test_mx_e2m1_table_is_the_pages(golden):
    """Codes 0..7 with a unit scale decode to the printed E2M1 magnitudes,
    8..15 to their negatives; the largest is 6; a 32-block with an 8-bit
    scale costs 4.25 bits per element."""
    _, p = golden
    t = p["fp4_e2m1"]
    codes = np.array([[c | (c + 1) << 4 for c in range(0, 16, 2)] * 2], np.uint8)  # 32 nibbles 0..15, 0..15
    out = oracle.mx_dequantize(codes, np.array([[127]], np.uint8), 1, 32)[0]
    assert np.array_equal(out[:8], np.array(t["magnitudes"], f32))
    assert np.array_equal(out[8:16], -np.array(t["magnitudes"], f32))
    assert out.max() == t["max"] and t["block"] == 32
    assert oracle.effective_bits(4, t["scale_bits"], 0, t["block"]) == t["bits_per_element"]


def test_mx_exponent_is_the_smallest_fitting_power_of_two():
    """e is the smallest integer with amax <= 6 * 2^e (checked by brute force
    in exact arithmetic), clamped to the E8M0 range."""
    import math
    rng = np.random.default_rng(40)
    cases = [6.0, 3.0, 1.5, 0.75, 1.0, 7.0, 12.0, 2.0 ** -100, 1e-45, 3e38]
    for e in (-126, -20, -1, 0, 5, 100):
        v = math.ldexp(6.0, e)
        cases += [v, float(np.nextafter(f32(v), f32(np.inf))), float(np.nextafter(f32(v), f32(0)))]
    cases += list(np.exp(rng.uniform(-60, 60, 200)))
    for a in cases:
        a = float(f32(a))
        got = oracle.mx_exponent(a)
        e = -200
        while math.ldexp(6.0, e) < a:
            e += 1
        assert got == max(-127, min(127, e)), (a, got, e)
    assert oracle.mx_exponent(0.0) == -127


def test_mx_round_trip_of_representable_blocks():
    """Blocks of +-E2M1 * 2^e containing 6 * 2^e come back exactly."""
    rng = np.random.default_rng(41)
    for e in (-30, -3, 0, 2, 40):
        vals = rng.choice(E2M1, (3, 64)) * rng.choice([-1.0, 1.0], (3, 64))
        vals[:, 0], vals[:, 32] = 6.0, -6.0
        vals = np.ldexp(vals, e)
        w = _mx_block_rows(vals)
        codes, scales = oracle.mx_quantize(w)
        assert np.all(scales == e + 127)
        assert np.array_equal(oracle.mx_dequantize(codes, scales, 3, 64), vals.astype(f32))


def test_mx_ties_go_to_the_even_encoding():
    """Half-way values between neighbouring magnitudes: 0.25 -> 0, 0.75 -> 1,
    1.25 -> 1, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4 (even = mantissa bit 0)."""
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    want = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    row = np.zeros(32)
    row[0] = 6.0
    row[1:8] = mids
    row[8:15] = [-m for m in mids]
    out = oracle.mx_dequantize(*oracle.mx_quantize(_mx_block_rows([row])), 1, 32)[0]
    assert list(out[1:8]) == want
    assert list(out[8:15]) == [-v if v else 0.0 for v in want]


def test_mx_brute_force_nearest_and_zero_sign():
    """Random blocks: every element is the nearest signed grid value times
    2^e (ties to the even encoding), zeros are stored as +0 codes, and the
    error is at most 2^e."""
    from workloads import f32_to_bf16_bits, bf16_bits_to_f32
    rng = np.random.default_rng(42)
    x = rng.standard_normal((40, 256)) * np.exp(rng.uniform(-8, 8, (40, 1)))
    x[3, :32] = 0.0
    x[4, 5] = -1e-30
    w = f32_to_bf16_bits(x)
    xf = bf16_bits_to_f32(w).astype(np.float64)
    codes, scales = oracle.mx_quantize(w)
    out = oracle.mx_dequantize(codes, scales, 40, 256).astype(np.float64)
    nib = _nibbles(codes, 256)
    e = scales.astype(np.int64).repeat(32, axis=1) - 127
    v = np.ldexp(xf, -e)
    grid = np.concatenate([-E2M1[::-1], E2M1])          # -6 .. 6
    enc = np.concatenate([np.arange(7, -1, -1), np.arange(8)])
    d = np.abs(v[..., None] - grid)
    dmin = d.min(-1)
    assert np.all(dmin <= 1.0)
    q = np.ldexp(out, -e)
    for idx in zip(*np.nonzero(np.abs(np.abs(v - q) - dmin) > 0)):
        raise AssertionError(f"not nearest at {idx}")
    tie = (np.isclose(d, dmin[..., None], rtol=0, atol=0)).sum(-1) > 1
    assert np.all((np.abs(q[tie]) == 0) | ((enc[np.searchsorted(grid, q[tie])] & 1) == 0))
    assert np.all(nib[out == 0] == 0)
    assert np.all(np.abs(out - xf) <= np.ldexp(1.0, e) + 0.0)


def test_mx_matmul_is_x_times_dequantized_transpose():
    from workloads import f32_to_bf16_bits, bf16_bits_to_f32
    rng = np.random.default_rng(43)
    n, k, m = 17, 320, 3
    w = f32_to_bf16_bits(rng.standard_normal((n, k)) * 0.02)
    x = f32_to_bf16_bits(rng.standard_normal((m, k)))
    codes, scales = oracle.mx_quantize(w)
    y = oracle.mx_matmul(x, codes, scales, n, k)
    ref = bf16_bits_to_f32(x).astype(np.float64) @ oracle.mx_dequantize(codes, scales, n, k).astype(np.float64).T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)
    full = bf16_bits_to_f32(x).astype(np.float64) @ bf16_bits_to_f32(w).astype(np.float64).T
    assert np.linalg.norm(y - full) / np.linalg.norm(full) < 0.2


# --------------------------------------------------------------------------
# GPTQ ("3.6 Quantization", GPTQ section).
# --------------------------------------------------------------------------
def _gptq_case(seed, t, n, k, corr=0.9):
    """Calibration X with correlated channels (a random mixing matrix), so
    that H is far from diagonal and compensation has something to do."""
    from workloads import f32_to_bf16_bits
    rng = np.random.default_rng(seed)
    base = rng.standard_normal((t, k))
    mix = np.eye(k) + corr * rng.standard_normal((k, k)) / np.sqrt(k)
    x = f32_to_bf16_bits(base @ mix)
    w = f32_to_bf16_bits(rng.standard_normal((n, k)) * 0.02)
    return x, w


def test_gptq_hessian_is_two_xtx():
    from workloads import bf16_bits_to_f32
    x, _ = _gptq_case(50, 24, 4, 128)
    xf = bf16_bits_to_f32(x).astype(np.float64)
    assert np.allclose(oracle.gptq_hessian(x), 2 * xf.T @ xf, rtol=1e-13, atol=1e-12)


def test_gptq_inverse_factor_is_the_cholesky_factor_of_the_inverse():
    """U is upper triangular with U^T U = (damped H)^-1; the damping adds 1 %
    of the mean diagonal (H of 24 tokens over 128 channels is singular)."""
    x, _ = _gptq_case(51, 24, 4, 128)
    h = oracle.gptq_hessian(x)
    hd, u = oracle.gptq_inverse_factor(h, 0.01)
    assert np.allclose(np.diag(hd) - np.diag(h), 0.01 * np.mean(np.diag(h)), rtol=1e-12)
    assert np.all(np.tril(u, -1) == 0) and np.all(np.diag(u) > 0)
    inv = np.linalg.inv(hd)
    ud = u.astype(np.float64)
    assert np.linalg.norm(ud.T @ ud - inv) / np.linalg.norm(inv) < 1e-5
    # and it is the Cholesky factor (unique with a positive diagonal)
    assert np.allclose(ud, np.linalg.cholesky(inv).T, rtol=1e-4, atol=1e-6 * np.abs(ud).max())


@pytest.mark.parametrize("symmetric", [False, True])
def test_gptq_with_a_multiple_of_the_identity_is_plain_rtn(symmetric):
    """H = c I makes U diagonal, so no column moves another: the codes are
    exactly the RTN codes of the original weights."""
    _, w = _gptq_case(52, 8, 6, 256)
    _, u = oracle.gptq_inverse_factor(3.0 * np.eye(256), 0.01)
    got = oracle.gptq_quantize(w, u, 4, symmetric, 128)
    want = oracle.quantize(w, 4, symmetric, 128)
    for g, r in zip(got, want):
        if r is not None:
            assert np.array_equal(g, r)


def _gptq_numpy(w_f32, hd, bits, symmetric, group):
    """The pages' update with explicit inverses of the remaining submatrix, in
    fp64: W_F -= e_j / [H_F^-1]_jj [H_F^-1]_{j,F}, then H_F^-1 loses row and
    column j (the block-inverse downdate). Returns the codes per column."""
    n, k = w_f32.shape
    qmax = 2 ** (bits - 1) - 1
    qmaxu = 2 ** bits - 1
    codes = np.zeros((n, k), np.int64)
    for r in range(n):
        w = w_f32[r].astype(np.float64)
        hinv = np.linalg.inv(hd)
        for j in range(k):
            if j % group == 0:
                g = w[j:j + group].astype(np.float32).astype(np.float64)
                if symmetric:
                    s = max(np.abs(g).max(), 1e-8) / qmax
                    z = 0.0
                else:
                    mn, mx = g.min(), g.max()
                    s = max(mx - mn, 1e-8) / qmaxu
                    z = np.round(-mn / s)
            q = np.clip(np.round(w[j] / s), -qmax, qmax) if symmetric else np.clip(np.round(w[j] / s) + z, 0, qmaxu)
            codes[r, j] = q
            e = w[j] - (q - z) * s
            w[j + 1:] -= e / hinv[j, j] * hinv[j, j + 1:]
            hinv = hinv - np.outer(hinv[:, j], hinv[j, :]) / hinv[j, j]
    return codes


def test_gptq_matches_the_explicit_inverse_formula():
    """The Cholesky-form fp32 oracle against the pages' formula in fp64:
    near-ties aside (fp32 vs fp64 sums), the codes are the same."""
    from workloads import bf16_bits_to_f32
    x, w = _gptq_case(53, 64, 6, 256)
    hd, u = oracle.gptq_inverse_factor(oracle.gptq_hessian(x), 0.01)
    codes, _, _ = oracle.gptq_quantize(w, u, 4, False, 128)
    got = _unpack4(codes, 256)
    want = _gptq_numpy(bf16_bits_to_f32(w), hd, 4, False, 128)
    assert np.mean(got == want) >= 0.995


def test_gptq_lowers_the_output_error_against_rtn():
    """The GPTQ section's claim: compensating each rounding error in the
    columns not yet quantized lowers ||W X - W_hat X|| on the calibration
    data against rounding every weight on its own."""
    from workloads import bf16_bits_to_f32
    x, w = _gptq_case(54, 96, 16, 256)
    n, k = 16, 256
    hd, u = oracle.gptq_inverse_factor(oracle.gptq_hessian(x), 0.01)
    xf = bf16_bits_to_f32(x).astype(np.float64)
    wf = bf16_bits_to_f32(w).astype(np.float64)
    def out_err(c, s, z):
        w_hat = oracle.dequantize(c, s, z, n, k, 4, False, 128).astype(np.float64)
        return np.linalg.norm(xf @ (wf - w_hat).T)
    e_gptq = out_err(*oracle.gptq_quantize(w, u, 4, False, 128))
    e_rtn = out_err(*oracle.quantize(w, 4, False, 128))
    assert e_gptq < 0.8 * e_rtn
