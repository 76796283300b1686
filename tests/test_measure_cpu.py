"""CPU checks of the benchmark's bookkeeping: byte counts and the
alpha-beta fit."""
import numpy as np

from collective_communication_ring_amd import measure


def test_fit_recovers_alpha_beta():
    n = np.array([2.0 ** k for k in range(3, 31)])
    alpha, beta = 12e-6, 1.0 / 300e9
    t = alpha + beta * n
    f = measure.fit_alpha_beta(n, t)
    assert abs(f["alpha_us"] - 12.0) < 1e-6
    assert abs(f["inv_beta_GBps"] - 300.0) < 1e-6
    assert f["max_rel_residual"] < 1e-9 and f["r2"] > 0.999999


def test_fit_with_noise_is_close():
    rng = np.random.default_rng(0)
    n = np.array([2.0 ** k for k in range(3, 31)])
    t = (5e-6 + n / 200e9) * (1 + 0.02 * rng.standard_normal(n.size))
    f = measure.fit_alpha_beta(n, t)
    assert abs(f["alpha_us"] - 5.0) < 0.5
    assert abs(f["inv_beta_GBps"] - 200.0) < 20.0


def test_byte_counts():
    # R = 8, fp32, 64 MiB per rank: 35 x 64 MiB
    assert measure.allreduce_alg_bytes(8, 16_777_216, 4) == 2_348_810_240
    # R = 16, bf16, 13,107,200 per rank: (10R - 14) N for reduce-scatter
    N = 13_107_200
    assert measure.reduce_scatter_alg_bytes(16, N, 2) == (10 * 16 - 14) * N
    assert measure.all_gather_alg_bytes(16, N, 2) == 2 * N * 2 + 4 * 15 * N
    # float32 reduce-scatter: every step reads 8 and writes 4 bytes
    assert measure.reduce_scatter_alg_bytes(8, 1024, 4) == 7 * 12 * 1024
    assert measure.reduce_scatter_alg_bytes(2, 1024, 4) == 12 * 1024
    # bf16 all-reduce with float32 partials: the reduce-scatter's (10R - 14) N,
    # then R - 1 copy steps of 2 bf16 each; with partials in T (acc = s) the
    # same count is 5 (R - 1) N s at every R
    assert measure.allreduce_alg_bytes(16, N, 2, acc=4) == (10 * 16 - 14) * N + 4 * 15 * N
    for R in (2, 3, 8, 16):
        assert measure.allreduce_alg_bytes(R, 1000, 2) == 5 * (R - 1) * 1000 * 2
        assert measure.allreduce_alg_bytes(R, 1000, 4, acc=4) == 5 * (R - 1) * 1000 * 4
    assert abs(measure.busbw_factor("allreduce", 8) - 1.75) < 1e-12
    assert abs(measure.busbw_factor("rs", 16) - 15 / 16) < 1e-12


def test_hbm_byte_counts():
    # R = 8 fp32 64 MiB per rank: 8 rows read + 8 rows written = 1 GiB
    assert measure.allreduce_hbm_bytes(8, 16_777_216, 4) == 1 << 30
    # R = 16 bf16 25 MiB buckets: 400 MiB read + 25 MiB written, and back
    N = 13_107_200
    assert measure.reduce_scatter_hbm_bytes(16, N, 2) == 425 << 20
    assert measure.all_gather_hbm_bytes(16, N, 2) == 425 << 20


def test_crossover_of_two_lines():
    # tree: 8 us + n / 20 GB/s; ring: 20 us + n / 200 GB/s -> equal at
    # n = 12 us / (1/20 - 1/200) us per kB = 266,666.7 bytes
    tree = dict(alpha_us=8.0, inv_beta_GBps=20.0)
    ring = dict(alpha_us=20.0, inv_beta_GBps=200.0)
    n = measure.crossover_bytes(tree, ring)
    assert abs(n - 12.0 / (1e-3 / 20 - 1e-3 / 200)) < 1e-6
    assert abs((8.0 + n * 1e-3 / 20) - (20.0 + n * 1e-3 / 200)) < 1e-9
    # a ring that is cheaper at every size never crosses
    assert measure.crossover_bytes(tree, dict(alpha_us=5.0, inv_beta_GBps=300.0)) is None
