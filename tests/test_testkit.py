"""The seeded input generators: published test vector, determinism, exact
outlier counts and the workload recipes."""
import numpy as np

import testkit


def test_splitmix64_reference_vector():
    # SplitMix64 from state 1234567: the reference outputs published with the
    # generator (Vigna's splitmix64.c; Java's SplittableRandom mixing).
    want = [6457827717110365317, 3203168211198807973, 9817491932198370423,
            4593380528125082431, 16408922859458223821]
    assert [testkit.lib().synth_draw(1234567, k) for k in range(5)] == want


def test_fill_independent_of_thread_count():
    a = testkit.fill((300, 1000), testkit.STUDENT_T3, 0.5, 99, threads=1)
    b = testkit.fill((300, 1000), testkit.STUDENT_T3, 0.5, 99, threads=7)
    np.testing.assert_array_equal(a, b)


def test_normal_moments():
    x = testkit.bf16_to_f32(testkit.fill((1 << 20,), testkit.NORMAL, 1.0, 5)).astype(np.float64)
    assert abs(x.mean()) < 5e-3 and abs(x.std() - 1) < 5e-3


def test_sample_is_exact_count_and_distinct():
    idx = testkit.sample(42, 10_000, 1_000)
    assert idx.size == 1000 and np.unique(idx).size == 1000
    assert idx.min() >= 0 and idx.max() < 10_000


def test_workload_recipes_small():
    x1 = testkit.make(1)
    assert x1.shape == (256, 1024)
    f = np.abs(testkit.bf16_to_f32(x1))
    assert 1100 <= (f > 6).sum() <= 1311  # 1311 entries were multiplied by 50
    x2 = testkit.make(2, rows=512)
    f2 = np.abs(testkit.bf16_to_f32(x2))
    col_max = f2.max(axis=0)
    assert (col_max > 40).sum() == 4  # 4 outlier channels x60
    x4 = testkit.make(4, rows=256)
    f4 = np.abs(testkit.bf16_to_f32(x4))
    assert (np.median(f4, axis=0) > 10).sum() == 8  # 8 outlier channels x100
    assert testkit.fnv1a64(x1) == testkit.fnv1a64(testkit.make(1))
