"""Pins of the oracle's decoded-weight matmul and activation rotation.

decode_matmul is the plain definition (decode, then multiply).  The pins tie
it to what the mathematics fixes: the rotation is orthogonal, so the same
product follows from the rotated activations and the looked-up pairs without
inverting the rotation; unit activations read single weights; the rotation
of activations preserves norms and has the closed form of the b = 2 case.
"""
import numpy as np
import pytest

import workloads
from oracle import qamw_ref as O


def _coded(N=6, d=64, b=16, K=16, seed=3, alpha=0.5):
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((N, d)) * 0.02
    r = rng.lognormal(0.0, 1.0, d)
    C = workloads.gaussian_samples(K, seed + 1).astype(np.float32)   # any codebook will do
    s, sigma, _ = O.calibrate(W, r, alpha, b, seed)
    enc = O.encode(W, s, sigma, b, seed, C)
    return dict(W=W, s=s, sigma=sigma, C=C, b=b, seed=seed, d=d, packed=enc["packed"], rn=enc["rho_hat_bits"])


def test_rotated_form_equals_definition():
    """rho^_n <R_fwd(X_t/s), y^_n> (no inverse rotation) == X W^^T (decode, then multiply)."""
    c = _coded()
    X = np.random.default_rng(9).standard_normal((5, c["d"]))
    Y = O.decode_matmul(X, c["packed"], c["rn"], c["s"], c["sigma"], c["b"], c["seed"], c["C"], c["d"])
    Xt = O.rotate_activations(X, c["s"], c["b"], c["seed"])
    Yh = O.lookup_pairs(c["packed"], c["sigma"], c["C"], c["d"])
    rho_hat = O.f16_bits_to_f64(c["rn"])
    Y2 = (Xt @ Yh.T) * rho_hat[None, :]
    assert np.allclose(Y, Y2, rtol=1e-12, atol=1e-15)


def test_without_s_uses_scaled_weights():
    c = _coded(seed=5)
    X = np.random.default_rng(1).standard_normal((3, c["d"]))
    Y = O.decode_matmul(X, c["packed"], c["rn"], None, c["sigma"], c["b"], c["seed"], c["C"], c["d"])
    Xt = O.rotate_activations(X, None, c["b"], c["seed"])
    Yh = O.lookup_pairs(c["packed"], c["sigma"], c["C"], c["d"])
    assert np.allclose(Y, (Xt @ Yh.T) * O.f16_bits_to_f64(c["rn"])[None, :], rtol=1e-12, atol=1e-15)


def test_unit_activation_reads_a_weight_column():
    c = _coded(seed=7)
    Wh = O.decode(c["packed"], c["rn"], c["s"], c["sigma"], c["b"], c["seed"], c["C"], c["d"])
    for j in (0, 5, 63):
        X = np.zeros((1, c["d"]))
        X[0, j] = 1.0
        Y = O.decode_matmul(X, c["packed"], c["rn"], c["s"], c["sigma"], c["b"], c["seed"], c["C"], c["d"])
        assert np.array_equal(Y[0], Wh[:, j])


def test_rotation_of_activations_is_orthogonal():
    rng = np.random.default_rng(2)
    X = rng.standard_normal((4, 256))
    Xt = O.rotate_activations(X, None, 128, 11)
    assert np.allclose(np.linalg.norm(Xt, axis=1), np.linalg.norm(X, axis=1), rtol=1e-13)


def test_rotation_of_activations_b2_closed_form():
    """b = 2: (x0 e0 + x1 e1, x0 e0 - x1 e1) / sqrt(2) per pair of columns."""
    X = np.array([[3.0, -1.0, 0.5, 2.0]])
    s = np.array([1.0, 2.0, 0.5, 4.0])
    eps = O.sign_mask(17, 4)
    Xt = O.rotate_activations(X, s, 2, 17)
    v = eps * X[0] / s
    ref = np.array([v[0] + v[1], v[0] - v[1], v[2] + v[3], v[2] - v[3]]) / np.sqrt(2)
    assert np.allclose(Xt[0], ref, rtol=1e-15, atol=1e-15)


def test_lookup_pairs_reads_codebook():
    C = np.array([[0.5, -1.0], [2.0, 0.25], [-3.0, 1.5], [0.0, 4.0]], np.float32)
    idx = np.array([[3, 0], [1, 2]])
    packed = O.pack(idx, 4, 4)
    sigma = np.array([2.0, 0.5])
    Yh = O.lookup_pairs(packed, sigma, C, 4)
    assert np.array_equal(Yh, [[0.0, 8.0, 0.25, -0.5], [4.0, 0.5, -1.5, 0.75]])
