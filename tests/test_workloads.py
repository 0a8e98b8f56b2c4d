"""Host-side checks of the seeded input generators (no method arithmetic)."""
import numpy as np

from workloads import (WORKLOADS, WORKLOAD_ORDER, bf16_bits_to_f32, f32_to_bf16_bits,
                       normal_bf16, normal_bf16_rows, CHUNK_ROWS)


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.0 - 2 ** -7, 3.0e38, 1e-40], np.float32)
    h = f32_to_bf16_bits(x)
    back = bf16_bits_to_f32(h)
    assert back[0] == 1.0
    assert back[1] == 1.0                      # tie -> even mantissa
    assert back[2] == 1.0 + 2 ** -6            # tie -> even (up)
    assert back[3] == -2.0                     # tie -> even
    assert np.isfinite(back[4])
    assert np.all(np.abs(back[:5] - x[:5]) <= np.abs(x[:5]) * 2 ** -8)
    assert abs(float(back[5]) - 1e-40) <= 2.0 ** -134   # bf16 subnormal spacing 2^-133


def test_row_subsets_regenerate_identically():
    seed = (2026, 9, 0, 0, 0)
    full = normal_bf16(seed, 3 * CHUNK_ROWS + 17, 64, 0.02)
    idx = np.array([0, 5, CHUNK_ROWS, 2 * CHUNK_ROWS + 3, 3 * CHUNK_ROWS + 16, 1])
    assert np.array_equal(normal_bf16_rows(seed, full.shape[0], 64, idx, 0.02), full[idx])
    assert np.array_equal(normal_bf16(seed, full.shape[0], 64, 0.02, None, 300, 700), full[300:700])


def test_workload_shapes_and_outliers():
    assert [WORKLOADS[n].index for n in WORKLOAD_ORDER] == [0, 1, 2, 3, 4]
    w7 = WORKLOADS["llama7b_decode"]
    m = w7.weight_col_mult(0, 4, 4096)
    assert np.count_nonzero(m == 20.0) == 41        # 1% of 4096 input channels x20
    m = w7.weight_col_mult(0, 6, 11008)
    assert np.count_nonzero(m == 20.0) == 110
    pf = WORKLOADS["prefill70b"]
    cm = pf.act_col_mult(8192)
    assert sorted(cm[cm > 1].tolist()) == [20.0, 28.0, 36.0, 44.0, 52.0, 60.0]
    sq = WORKLOADS["smoothquant"]
    cm = sq.act_col_mult(8192)
    assert np.count_nonzero(cm == 50.0) == 6
    w70 = WORKLOADS["llama70b_decode"]
    assert [(l.n, l.k) for l in w70.linears] == [(8192, 8192), (1024, 8192), (1024, 8192), (8192, 8192),
                                                 (28672, 8192), (28672, 8192), (8192, 28672)]


def test_weight_statistics():
    w = bf16_bits_to_f32(WORKLOADS["single_4096"].weight(0, 0, rows=np.arange(64)))
    assert abs(w.std() - 0.02) < 0.001 and abs(w.mean()) < 0.001
