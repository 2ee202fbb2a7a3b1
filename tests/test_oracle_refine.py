"""Pins of the codebook refinement on a matrix's own pairs
(oracle/lloyd.py: refine_on_pairs): closed forms and Lloyd's monotonicity."""
import os

import numpy as np

import workloads
from oracle import lloyd
from oracle import qamw_ref as O

CB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                  "vector_codebook_codec_amd", "codebooks")


def test_one_centroid_moves_to_the_mean():
    Z = np.random.default_rng(1).standard_normal((999, 2)) + [0.3, -1.2]
    C, hist = lloyd.refine_on_pairs(Z, np.array([[5.0, 5.0]], np.float32), 1)
    assert np.allclose(C[0], Z.mean(axis=0).astype(np.float32), atol=0)
    assert abs(hist[0] - np.mean(np.sum((Z - [5.0, 5.0]) ** 2, axis=1))) < 1e-12


def test_two_separated_clusters():
    rng = np.random.default_rng(2)
    A = rng.standard_normal((300, 2)) * 0.1 + [-3, 0]
    B = rng.standard_normal((200, 2)) * 0.1 + [3, 0]
    C, hist = lloyd.refine_on_pairs(np.concatenate([A, B]), np.array([[-1, 0], [1, 0]], np.float32), 2)
    assert np.allclose(C[0], A.mean(0), atol=1e-6) and np.allclose(C[1], B.mean(0), atol=1e-6)
    assert hist[1] < hist[0]


def test_empty_cell_keeps_its_centroid_and_points_on_centroids_cost_nothing():
    C0 = np.array([[0, 0], [1, 0], [50, 50]], np.float32)
    Z = np.array([[0, 0], [1, 0], [0, 0], [1, 0]], np.float64)
    C, hist = lloyd.refine_on_pairs(Z, C0, 1)
    assert np.array_equal(C, C0) and hist[0] == 0.0


def test_distortion_never_increases_on_matrix_pairs():
    wl = workloads.get("c1_256x512")
    s, sig, _ = O.calibrate(wl.W_f32(), wl.r, wl.alpha, wl.block, wl.sign_seed)
    Zt, _ = O.normalized_pairs(wl.W_f32(), s, sig, wl.block, wl.sign_seed)
    C0 = np.fromfile(os.path.join(CB, "qamw_K256.f32"), dtype="<f4").reshape(-1, 2)
    C, hist = lloyd.refine_on_pairs(Zt.reshape(-1, 2), C0, 6)
    assert all(b <= a + 1e-12 for a, b in zip(hist, hist[1:]))
    assert hist[-1] < hist[0]
