"""The seeded input generator (CPU only)."""
import numpy as np

from delta_rule_linear_amd import inputs


def test_bf16_round_to_nearest_even():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1) wins;
    # 1 + 3*2^-8 ties between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -2.5, 0.0], np.float32)
    want = np.array([1.0, 1 + 2 ** -6, 1 + 2 ** -7, -2.5, 0.0], np.float32)
    assert np.array_equal(inputs.round_bf16(x), want)
    assert np.array_equal(inputs.bf16_bits(want)[:1], np.array([0x3F80], np.uint16))


def test_small_problem_shapes_and_recipe():
    p = inputs.make_chunk_problem(2, 3, 70, 64, 64, gate="channel", beta_mode="channel",
                                  log_alpha_range=(-0.2, -0.0005), s0_var=0.01, seed=0)
    assert p.q.shape == (2, 3, 70, 64) and p.log_alpha.shape == (2, 3, 70, 64)
    assert p.beta.shape == (2, 3, 70, 64) and p.S0.shape == (2, 3, 64, 64)
    # bf16-exact, and unit norm up to bf16 rounding
    inputs.bf16_bits(p.q)
    n = np.linalg.norm(p.k.astype(np.float64), axis=-1)
    assert np.all(np.abs(n - 1) < 2 ** -7)
    assert p.log_alpha.min() >= -0.2 and p.log_alpha.max() <= -0.0005
    assert 0 < p.beta.min() and p.beta.max() < 1
    assert abs(p.S0.std() - 0.1) < 0.01
    q = inputs.make_chunk_problem(2, 3, 70, 64, 64, gate="channel", beta_mode="channel",
                                  log_alpha_range=(-0.2, -0.0005), s0_var=0.01, seed=0)
    assert np.array_equal(p.v, q.v) and np.array_equal(p.S0, q.S0)


def test_workload_table():
    w = inputs.WORKLOADS
    assert w["gdn_b2h16_16k"]["L"] == 16384 and w["gdn_b2h16_16k"]["gate"] == "scalar"
    assert w["fg2_b2h16_16k"]["beta_mode"] == "channel"
    small = inputs.workload("deltanet_f32")
    assert small.q.dtype == np.float32 and small.log_alpha is None and small.S0 is None


def test_decode_problem_small():
    d = inputs.make_decode_problem(N=4, H=2, Dk=64, Dv=64, steps=3)
    assert d.S.shape == (4, 2, 64, 64) and d.q.shape == (3, 4, 2, 64)
    assert d.log_alpha.shape == (3, 4, 2) and d.beta.shape == (3, 4, 2)
