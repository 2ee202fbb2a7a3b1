"""The seeded input generators (CPU): determinism, shapes, bf16 rounding."""
import numpy as np

import workloads


def test_bf16_rounding_pins():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0, 1.0 + 2 ** -8 + 2 ** -20],
                    dtype=np.float32)
    got = workloads.bf16_bits_to_f32(workloads.bf16_bits_from_f32(vals))
    assert list(got) == [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 0.0, 1.0 + 2 ** -7]
    assert workloads.bf16_bits_from_f32(np.array([1.0], np.float32))[0] == 0x3F80


def test_c1_shape_and_determinism():
    a = workloads.get("c1_256x512")
    b = workloads.get("c1_256x512")
    assert a.W.shape == (256, 512) and a.W.dtype == np.float32
    assert np.array_equal(a.W, b.W) and np.array_equal(a.r, b.r)
    assert abs(a.W.std() - 0.02) < 0.001 and np.all(a.r > 0)
    assert (a.alpha, a.block, a.sign_seed, a.K) == (0.5, 128, 0, 256)


def test_outlier_columns():
    W = workloads.matrix(64, 400, dist="normal", std=0.02, seed=5,
                         outlier_frac=0.01, outlier_scale=8.0, outlier_seed=6)
    col_sd = W.std(axis=0)
    assert (col_sd > 0.08).sum() == 4


def test_t5_scale():
    W = workloads.matrix(512, 512, dist="t5", std=0.02, seed=7)
    assert abs(W.std() - 0.02) < 0.001


def test_names_resolve():
    for n in workloads.names():
        assert n.startswith("c")
    assert workloads.stack_7b(0, "down").name == "c5_l0_down"
