"""Pins of the output-error oracle (oracle/output_error.py): the pages' trace
identity evaluated the other way round, special activations with closed
forms, scaling laws, and the Cauchy-Schwarz optimum of the channel-scale
exponent."""
import numpy as np
import pytest

import workloads
from oracle import output_error as E
from oracle import qamw_ref as O


def test_trace_identity_against_the_output_form():
    rng = np.random.default_rng(1)
    X = rng.standard_normal((37, 24)) * rng.lognormal(0, 1, 24)
    dW = rng.standard_normal((19, 24))
    direct = float(np.sum((X @ dW.T) ** 2))                      # || X dW^T ||_F^2
    assert abs(E.output_error(dW, np.zeros_like(dW), X) - direct) <= 1e-10 * direct


def test_identity_activations_give_the_frobenius_norm():
    rng = np.random.default_rng(2)
    W = rng.standard_normal((7, 16))
    Wh = W + 0.01 * rng.standard_normal((7, 16))
    assert abs(E.output_error(W, Wh, np.eye(16)) - np.sum((W - Wh) ** 2)) < 1e-14


def test_diagonal_activations_weight_columns():
    rng = np.random.default_rng(3)
    c = rng.uniform(0.5, 3.0, 12)
    dW = rng.standard_normal((5, 12))
    want = float(np.sum(c ** 2 * np.sum(dW ** 2, axis=0)))
    assert abs(E.output_error(dW, 0 * dW, np.diag(c)) - want) < 1e-12 * want


def test_scaling_laws_and_zero_error():
    rng = np.random.default_rng(4)
    X = rng.standard_normal((20, 8))
    W = rng.standard_normal((3, 8))
    Wh = W + rng.standard_normal((3, 8))
    e = E.output_error(W, Wh, X)
    assert e > 0
    assert abs(E.output_error(W, Wh, 3 * X) - 9 * e) < 1e-10 * e
    assert abs(E.output_error(2 * W, 2 * Wh, X) - 4 * e) < 1e-10 * e
    assert E.output_error(W, W, X) == 0.0


def test_channel_rms_closed_forms():
    X = np.tile(np.array([[1.5, -2.0, 0.0, 3.0]]), (10, 1))
    assert np.allclose(E.channel_rms(X), [1.5, 2.0, 0.0, 3.0], atol=1e-15)
    rng = np.random.default_rng(5)
    X = rng.standard_normal((50, 9))
    assert np.allclose(E.channel_rms(X) ** 2, np.diag(E.gram(X)) / 50, rtol=1e-13)
    M = E.gram(X)
    assert np.allclose(M, M.T) and np.linalg.eigvalsh(M).min() > -1e-10


def test_generated_activations_have_the_requested_rms():
    r = workloads.channel_rms(64, sigma_log=1.0, seed=6)
    X = workloads.activations(20000, r, seed=7)
    assert np.allclose(E.channel_rms(X), r, rtol=0.05)


@pytest.mark.parametrize("K", [256])
def test_alpha_half_minimises_the_output_error(K):
    """For i.i.d. weights the output error of the scaled codec behaves like
    (sum_j r_j^(2 alpha)) (sum_j r_j^(2 - 2 alpha)) (row norm times per-column
    error), which Cauchy-Schwarz minimises at alpha = 1/2."""
    rng = np.random.default_rng(8)
    N, d, b, seed = 64, 512, 128, 99
    W = rng.standard_normal((N, d)) * 0.02
    r = workloads.channel_rms(d, sigma_log=1.2, seed=9)
    X = workloads.activations(256, r, seed=10)
    rx = E.channel_rms(X)
    import os
    C = np.fromfile(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                                 "vector_codebook_codec_amd", "codebooks", f"qamw_K{K}.f32"),
                    dtype="<f4").reshape(-1, 2)
    err = {}
    for alpha in (0.0, 0.5, 1.0):
        s, sig, _ = O.calibrate(W, rx, alpha, b, seed)
        enc = O.encode(W, s, sig, b, seed, C)
        Wh = O.decode(enc["packed"], enc["rho_hat_bits"], s, sig, b, seed, C, d)
        err[alpha] = E.output_error(W, Wh, X)
    assert err[0.5] < err[0.0] and err[0.5] < err[1.0], err
