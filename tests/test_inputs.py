"""Seeded input generator: determinism, bf16 rounding and the workload table."""

import numpy as np

from software_pipelined_amd import inputs as I


def test_bf16_round_to_nearest_even_bit_patterns():
    f = np.array([
        1.0,                 # exact
        -2.0,                # exact, sign
        0.0, -0.0,
        1.0 + 2.0 ** -8,     # halfway between 1 and 1+2^-7: ties to even -> 1.0
        1.0 + 3 * 2.0 ** -8,  # halfway, odd lower neighbour -> rounds up to 1+2^-6
        1.0 + 2.0 ** -8 + 2.0 ** -20,  # just above halfway -> up
        3.0e38,              # large finite
        1.0e-40,             # float32 subnormal
    ], dtype=np.float32)
    got = I.f32_to_bf16_bits(f)
    want = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x3F80, 0x3F82, 0x3F81, 0x7F62, 0x0001],
                    dtype=np.uint16)
    np.testing.assert_array_equal(got, want)
    # widening is exact and round-trips
    np.testing.assert_array_equal(I.f32_to_bf16_bits(I.bf16_bits_to_f32(want)), want)


def test_generator_is_deterministic_and_seeded():
    a = I.gen_qkv(1, 2, 33, 64, seed=5)
    b = I.gen_qkv(1, 2, 33, 64, seed=5)
    c = I.gen_qkv(1, 2, 33, 64, seed=6)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    assert not np.array_equal(a[0], c[0])
    q, k, v = a
    assert q.dtype == np.uint16 and q.shape == (1, 2, 33, 64) and q.flags.c_contiguous
    qf = I.bf16_bits_to_f32(q)
    assert abs(float(qf.mean())) < 0.1 and 0.9 < float(qf.std()) < 1.1


def test_key_stress_scales_every_seventh_key_exactly():
    q0, k0, v0 = I.gen_qkv(1, 1, 30, 16, seed=3)
    q1, k1, v1 = I.gen_qkv(1, 1, 30, 16, seed=3, key_stress=True)
    np.testing.assert_array_equal(q0, q1)
    np.testing.assert_array_equal(v0, v1)
    kf0, kf1 = I.bf16_bits_to_f32(k0), I.bf16_bits_to_f32(k1)
    rows = np.arange(30)
    np.testing.assert_array_equal(kf1[:, :, rows % 7 == 0], 8 * kf0[:, :, rows % 7 == 0])
    np.testing.assert_array_equal(kf1[:, :, rows % 7 != 0], kf0[:, :, rows % 7 != 0])


def test_workload_table_and_flop_counts():
    names = [c.name for c in I.CONFIGS]
    assert len(set(names)) == 5
    h = I.HEADLINE
    assert (h.B, h.H, h.N, h.d, h.causal) == (2, 16, 16384, 128, False)
    assert h.flops() == 4 * 2 * 16 * 128 * 16384 ** 2
    c = I.CAUSAL_2K
    assert c.visible_pairs_per_head() == 2048 * 2049 // 2
    assert I.default_scale(128) == np.float32(1.0 / np.sqrt(128.0))
    assert I.default_scale(64) == np.float32(0.125)


def test_sample_rows_cover_every_head_and_edges():
    rows = I.sample_rows(2, 3, 1000, per_head=20, seed=1)
    assert rows.dtype == np.int64 and np.all(np.diff(rows) > 0)
    for bh in range(6):
        r = rows[(rows >= bh * 1000) & (rows < (bh + 1) * 1000)] - bh * 1000
        assert 0 in r and 999 in r and len(r) >= 20
