"""SmoothQuant path: smoothing scale, per-token INT8 and per-channel INT8
weights, bit-exact against the oracle."""
import numpy as np
import pytest

import bit_gemv_amd as bg
import oracle
from gpu_helpers import assert_same_bits, dev, dev_bf16, host, say
from workloads import f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def _xw(t, n, k, seed=0, outliers=6, mult=50.0):
    rng = np.random.default_rng(seed)
    xf = rng.standard_normal((t, k))
    idx = rng.choice(k, outliers, replace=False)
    xf[:, idx] *= mult
    wf = rng.standard_normal((n, k)) * 0.02
    return f32_to_bf16_bits(xf), f32_to_bf16_bits(wf)


@pytest.mark.parametrize("t,n,k", [(1, 1, 128), (7, 65, 384), (64, 300, 2048 + 128), (512, 1024, 8192)])
def test_smooth_scale_alpha_half(t, n, k):
    x, w = _xw(t, n, k, seed=t)
    say(f"smooth_scale t={t} n={n} k={k}")
    s = host(bg.smooth_scale(dev_bf16(x), dev_bf16(w), 0.5))
    assert_same_bits(s, oracle.smooth_scale(x, w, 0.5), "s")


def test_smooth_scale_rows_past_grid_extent():
    """More 64-row tiles of W than a grid's y extent (65535) holds: blocks
    stride over the rest. Large values planted in the last tile's rows must
    reach s."""
    n, k = 65535 * 64 + 70, 128
    x, w0 = _xw(4, 256, k, seed=5)
    w = np.tile(w0, (n // 256 + 1, 1))[:n].copy()
    big = f32_to_bf16_bits(np.array([3.0, -5.0, 7.0]))
    w[n - 1, 3], w[65535 * 64 + 5, 50], w[65535 * 64, 127] = big
    say(f"smooth_scale t=4 n={n} k={k}")
    s = host(bg.smooth_scale(dev_bf16(x), dev_bf16(w), 0.5))
    ref = oracle.smooth_scale(x, w, 0.5)
    assert ref[3] != oracle.smooth_scale(x, w[:65535 * 64], 0.5)[3]
    assert_same_bits(s, ref, "s")


@pytest.mark.parametrize("alpha", [0.0, 0.25, 0.8, 1.0])
def test_smooth_scale_other_alpha(alpha):
    x, w = _xw(33, 70, 1024, seed=2)
    say(f"smooth_scale alpha={alpha}")
    s = host(bg.smooth_scale(dev_bf16(x), dev_bf16(w), alpha))
    ref = oracle.smooth_scale(x, w, alpha)
    assert np.allclose(s, ref, rtol=1e-6, atol=0), np.abs(s / ref - 1).max()


def test_smooth_scale_zero_channels():
    x, w = _xw(8, 16, 256, seed=3)
    x[:, 10] = 0
    w[:, 11] = 0
    x[:, 12] = 0
    w[:, 12] = 0
    say("smooth_scale zero channels")
    s = host(bg.smooth_scale(dev_bf16(x), dev_bf16(w), 0.5))
    assert_same_bits(s, oracle.smooth_scale(x, w, 0.5), "s")


# A token's row is held in registers 8192 channels at a time: rows of one
# partial or full chunk, then 8320 and 28672 channels (two and four chunks,
# the earlier ones read again for their codes).
@pytest.mark.parametrize("smooth", [False, True])
@pytest.mark.parametrize("t,k", [(1, 128), (5, 384), (64, 2048 + 128), (512, 8192), (3, 8192 + 128), (7, 28672),
                                 (4, 16384), (2, 65536)])
def test_per_token_int8(t, k, smooth):
    x, w = _xw(t, 16, k, seed=k)
    sm = np.exp(np.random.default_rng(1).uniform(-2, 2, k)).astype(np.float32) if smooth else None
    say(f"quant_per_token_int8 t={t} k={k} smooth={smooth}")
    qx, sx = bg.quant_per_token_int8(dev_bf16(x), None if sm is None else dev(sm))
    q_ref, s_ref = oracle.quant_per_token_int8(x, sm)
    assert_same_bits(host(qx), q_ref, "qx")
    assert_same_bits(host(sx), s_ref, "sx")


def test_per_token_edge_rows():
    k = 256
    rows = [np.zeros(k), np.full(k, 2.5), np.linspace(-127, 127, k), np.full(k, 1e-39)]
    x = f32_to_bf16_bits(np.stack(rows))
    say("quant_per_token_int8 edge rows")
    qx, sx = bg.quant_per_token_int8(dev_bf16(x))
    q_ref, s_ref = oracle.quant_per_token_int8(x)
    assert_same_bits(host(qx), q_ref, "qx")
    assert_same_bits(host(sx), s_ref, "sx")


@pytest.mark.parametrize("k", [256, 8192])
def test_per_token_exact_ties_and_top_codes(k):
    """Rows aimed at the code placement. Exact rounding ties: the
    half-integers -126.5 .. 126.5 beside +-127, so s = 1 (and s = 2^-20 for
    the row times 2^-20) and X' / s is m + 1/2 exactly, which must round to
    the even neighbour. Rows whose scale s = RN(max|X'| / 127) rounded down,
    so the top quotient max|X'| / s lies just above 127 and must still give
    the code 127 (and -127 for its negative). 8192 channels (the 256 tiled)
    take the kernel's unguarded whole-chunk form, 256 the guarded one."""
    half = np.arange(-126.5, 127.0, 1.0)
    tie = np.concatenate([[127.0, -127.0], half])
    rows = [tie, tie * 2.0 ** -20]
    rng = np.random.default_rng(41)
    cand = oracle.bf16_bits_to_f32(f32_to_bf16_bits(rng.uniform(1e-3, 1e3, 4096)))
    s32 = cand / np.float32(127.0)
    down = cand[s32.astype(np.float64) < cand.astype(np.float64) / 127.0]
    assert len(down) >= 14
    for am in down[:14]:
        rows.append(np.concatenate([[am, -am], am * rng.uniform(-1.0, 1.0, 254)]))
    x = f32_to_bf16_bits(np.tile(np.stack(rows), (1, k // 256)))
    for sm in (None, np.ones(k, np.float32)):
        say(f"quant_per_token_int8 exact ties and top codes k={k} smooth={sm is not None}")
        qx, sx = bg.quant_per_token_int8(dev_bf16(x), None if sm is None else dev(sm))
        q_ref, s_ref = oracle.quant_per_token_int8(x, sm)
        assert_same_bits(host(sx), s_ref, "sx")
        assert_same_bits(host(qx), q_ref, "qx")
    # what the rows are for, on the oracle's side
    assert s_ref[0] == 1.0 and s_ref[1] == np.float32(2.0 ** -20)
    assert (q_ref[:2, 2:256] == np.rint(half).astype(np.int8)).all()
    assert (q_ref[:, 0] == 127).all() and (q_ref[:, 1] == -127).all()


def test_per_token_quotients_next_to_rounding_ties():
    """Smoothed activations X' placed within 0..3 fp32 ulps of (m + 1/2) s,
    with s = max|X'| / 127 of the token, so X' / s lands next to (or on) a
    half-way point: the codes decide between two integers there, and the
    division must be the IEEE one for them to agree bit for bit. Token i is
    token 0 times 2^(i - 2) (exact in bf16), so every token carries the same
    near-tie quotients at its own magnitude."""
    t, k = 6, 1024
    rng = np.random.default_rng(31)
    x0 = f32_to_bf16_bits(rng.uniform(1.0, 2.0, k)).astype(np.uint32) << 16
    x0 = x0.view(np.float32)
    xs = f32_to_bf16_bits(np.stack([x0 * np.float32(2.0 ** (i - 2)) for i in range(t)]))
    s0 = rng.uniform(0.5, 2.0)
    target = np.empty(k)
    target[0] = 127.0 * s0
    target[1:] = (rng.integers(-126, 126, k - 1) + 0.5) * s0
    ulps = rng.integers(-3, 4, k)
    ulps[0] = 0
    t32 = target.astype(np.float32)
    for j in range(1, k):
        for _ in range(abs(int(ulps[j]))):
            t32[j] = np.nextafter(t32[j], np.float32(np.inf if ulps[j] > 0 else -np.inf), dtype=np.float32)
    sm = (x0.astype(np.float64) / t32.astype(np.float64)).astype(np.float32)
    say("quant_per_token_int8 near-tie quotients")
    qx, sx = bg.quant_per_token_int8(dev_bf16(xs), dev(sm))
    q_ref, s_ref = oracle.quant_per_token_int8(xs, sm)
    assert_same_bits(host(sx), s_ref, "sx")
    assert_same_bits(host(qx), q_ref, "qx")


def test_smoothed_weight_quantization_chain():
    """s from the GPU, then W * s per-channel INT8 on both sides."""
    x, w = _xw(128, 256, 4096, seed=11)
    say("smoothquant weight chain")
    s_gpu = bg.smooth_scale(dev_bf16(x), dev_bf16(w), 0.5)
    s = host(s_gpu)
    assert_same_bits(s, oracle.smooth_scale(x, w, 0.5), "s")
    pw = bg.quantize_groupwise(dev_bf16(w), 8, True, 4096, s_gpu)
    c_ref, sw_ref, _ = oracle.quantize(w, 8, True, 4096, s)
    assert_same_bits(host(pw.codes), c_ref, "qw")
    assert_same_bits(host(pw.scales), sw_ref, "sw")
