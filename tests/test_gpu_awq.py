"""AWQ scale search on the GPU against the oracle on the same inputs.

Integer results (codes, and the channel magnitudes s_X, whose fp64 sums are
exact here) are compared bit for bit. The losses are float sums compared at
a relative tolerance; the chosen grid point must be the oracle's argmin or,
where two grid points are that close, one whose oracle loss is within the
tolerance of the minimum. s = powf(s_X, alpha) comes from the device's powf,
which may differ from the host's by an ulp, so the final codes are checked
against the oracle's quantizer run on the device's s_best.
"""
import numpy as np
import pytest

import bit_gemv_amd as bg
import oracle
from gpu_helpers import assert_same_bits, dev, dev_bf16, host, say
from workloads import WORKLOADS, f32_to_bf16_bits

pytestmark = pytest.mark.gpu

LOSS_RTOL = 1e-3


def _inputs(t, n, k, seed, outliers=(), mult=20.0, w_scale=0.02):
    rng = np.random.default_rng(seed)
    xf = rng.standard_normal((t, k)).astype(np.float32)
    if len(outliers):
        xf[:, list(outliers)] *= np.float32(mult)
    return f32_to_bf16_bits(xf), f32_to_bf16_bits(rng.standard_normal((n, k)) * w_scale)


@pytest.mark.parametrize("t,k", [(1, 128), (7, 200), (24, 384), (512, 4096 + 64), (333, 11008)])
def test_act_absmean_bit_exact(t, k):
    x, _ = _inputs(t, 1, k, seed=t + k, outliers=(0, k - 1), mult=30.0)
    say(f"act_absmean t={t} k={k}")
    sx = host(bg.act_absmean(dev_bf16(x)))
    assert_same_bits(sx, oracle.act_absmean(x), "sx")


def _check_search(x, w, symmetric, group, n_grid, what):
    t, k = x.shape
    n = w.shape[0]
    say(f"awq_search {what}: t={t} n={n} k={k} sym={symmetric} group={group} n_grid={n_grid}")
    r = bg.awq_search(dev_bf16(x), dev_bf16(w), symmetric=symmetric, group=group, n_grid=n_grid)
    losses, best, s_best = host(r.losses), int(host(r.best)[0]), host(r.s_best)
    sx_ref, l_ref, best_ref, _ = oracle.awq_search(x, w, 4, symmetric, group, n_grid)
    rel = np.abs(losses - l_ref) / l_ref
    say(f"  losses max rel diff {rel.max():.2e}; best gpu {best} oracle {best_ref} "
        f"(loss ratio best/alpha0 {l_ref[best_ref] / l_ref[0]:.3f})")
    assert np.all(rel <= LOSS_RTOL), rel
    assert best == best_ref or l_ref[best] <= l_ref.min() * (1 + LOSS_RTOL)
    # s_best is grid point `best` of the device's s_X (bit-exact with the oracle's)
    sx_dev = host(bg.act_absmean(dev_bf16(x)))
    assert_same_bits(sx_dev, sx_ref, "sx")
    s_host = oracle.awq_scale(sx_ref, best, n_grid)
    assert np.allclose(s_best, s_host, rtol=4e-7, atol=0), np.abs(s_best / s_host - 1).max()
    # the packed weights are the quantizer's output on W diag(s_best)
    c_ref, s_ref, z_ref = oracle.quantize(w, 4, symmetric, group, col_scale=s_best)
    assert_same_bits(host(r.packed.codes), c_ref, "codes")
    assert_same_bits(host(r.packed.scales), s_ref, "scales")
    if not symmetric:
        assert_same_bits(host(r.packed.zeros), z_ref, "zeros")
    return r, l_ref


@pytest.mark.parametrize("symmetric", [False, True])
@pytest.mark.parametrize("t,n,k", [(64, 200, 512), (13, 129, 384), (130, 64, 1024)])
def test_awq_search_matches_oracle(t, n, k, symmetric):
    """Ragged token and row counts (tails of the 128 x 128 product tiles),
    several groups per row, outlier channels."""
    x, w = _inputs(t, n, k, seed=t * n, outliers=(3, 100, k - 5), mult=25.0)
    _check_search(x, w, symmetric, 128, 20, "small")


@pytest.mark.parametrize("group", [256, "k"])
def test_awq_search_larger_groups(group):
    k = 768
    x, w = _inputs(40, 96, k, seed=9, outliers=(1, 500), mult=30.0)
    _check_search(x, w, False, k if group == "k" else group, 10, f"group {group}")


def test_awq_search_two_point_grid_and_one_token():
    x, w = _inputs(1, 48, 256, seed=4, outliers=(17,), mult=40.0)
    _check_search(x, w, False, 128, 1, "alpha in {0, 1}")


def test_awq_search_protects_outliers_and_is_repeatable():
    """The method's claim on outlier activations (alpha > 0 beats plain RTN),
    and two calls on one workspace give identical bits."""
    x, w = _inputs(96, 256, 1024, seed=21, outliers=(5, 77, 300, 811), mult=40.0)
    r, l_ref = _check_search(x, w, False, 128, 20, "outliers")
    assert int(host(r.best)[0]) > 0
    assert l_ref[int(host(r.best)[0])] < 0.8 * l_ref[0]
    import torch
    ws = torch.empty(bg.load_library().awq_workspace_bytes(96, 256, 1024), dtype=torch.uint8,
                        device="cuda")
    a = bg.awq_search(dev_bf16(x), dev_bf16(w), workspace=ws)
    b = bg.awq_search(dev_bf16(x), dev_bf16(w), workspace=ws)
    for u, v in ((a.losses, b.losses), (a.s_best, b.s_best), (a.packed.codes, b.packed.codes)):
        assert_same_bits(host(u), host(v), "repeat")


def test_awq_workload_layer_q_projection_properties():
    """The AWQ workload's q projection at full size (512 tokens, 4096 x 4096):
    channel magnitudes bit-exact, the loss curve has its minimum at the
    chosen grid point and beats plain RTN, s_best is that grid point's scale,
    and sampled rows of the packed weights equal the oracle's quantizer on
    W diag(s_best)."""
    wl = WORKLOADS["awq7b"]
    lin = wl.linears[0]
    x = wl.activation(lin.k, wl.tokens)
    w = wl.weight(0, 0)
    say(f"awq_search workload {wl.name} {lin.name} {lin.n}x{lin.k}, t={wl.tokens}")
    r = bg.awq_search(dev_bf16(x), dev_bf16(w), symmetric=wl.symmetric, group=wl.group,
                      n_grid=wl.extra["n_grid"])
    losses, best, s_best = host(r.losses), int(host(r.best)[0]), host(r.s_best)
    sx = oracle.act_absmean(x)
    assert_same_bits(host(bg.act_absmean(dev_bf16(x))), sx, "sx")
    assert best == int(np.argmin(losses))
    assert best > 0 and losses[best] < losses[0]
    assert np.allclose(s_best, oracle.awq_scale(sx, best, wl.extra["n_grid"]), rtol=4e-7, atol=0)
    rows = np.random.default_rng(0).choice(lin.n, 64, replace=False)
    c_ref, s_ref, z_ref = oracle.quantize(w[rows], 4, wl.symmetric, wl.group, col_scale=s_best)
    assert_same_bits(host(r.packed.codes)[rows], c_ref, "codes (sampled rows)")
    assert_same_bits(host(r.packed.scales)[rows], s_ref, "scales (sampled rows)")
    assert_same_bits(host(r.packed.zeros)[rows], z_ref, "zeros (sampled rows)")
