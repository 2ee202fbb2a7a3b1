"""Pins for the oracle's sign mask and rotation (CPU only).

The rotation is a sign-masked block Hadamard transform that is an exact
isometry (QAM-W, Methodology, Deterministic Rotation).  The pins below come
from outside the oracle: published SplitMix64 outputs, SciPy's Sylvester
Hadamard construction, an independent butterfly FWHT written here, the
closed form for b = 2 and orthogonality.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg

from conftest import GOLDEN
from oracle import qamw_ref as Q


def test_splitmix64_published_vectors():
    with open(os.path.join(GOLDEN, "splitmix64_seed1234567.json")) as f:
        g = json.load(f)
    got = Q.splitmix64(g["seed"], len(g["outputs"]))
    assert got == [int(v) for v in g["outputs"]]


def test_sign_mask_bit63_and_balance():
    outs = Q.splitmix64(7, 4096)
    eps = Q.sign_mask(7, 4096)
    assert set(np.unique(eps)) <= {-1.0, 1.0}
    assert np.array_equal(eps < 0, np.array([v >= (1 << 63) for v in outs]))
    # a fair coin over 4096 draws: 6 standard deviations
    assert abs((eps < 0).mean() - 0.5) < 6 * 0.5 / math.sqrt(4096)
    # different seeds give different masks; a prefix of a longer mask is the shorter mask
    assert not np.array_equal(Q.sign_mask(0, 256), Q.sign_mask(1, 256))
    assert np.array_equal(Q.sign_mask(3, 100), Q.sign_mask(3, 300)[:100])


@pytest.mark.parametrize("b", [1, 2, 4, 8, 16, 64, 128, 256, 1024])
def test_sylvester_matches_scipy(b):
    assert np.array_equal(Q.sylvester_hadamard(b), scipy.linalg.hadamard(b).astype(np.float64))


def _fwht_butterfly(v):
    """Independent in-place iterative Walsh-Hadamard butterfly (natural order)."""
    a = np.array(v, dtype=np.float64)
    n = a.shape[-1]
    h = 1
    while h < n:
        for i in range(0, n, 2 * h):
            x = a[..., i:i + h].copy()
            y = a[..., i + h:i + 2 * h].copy()
            a[..., i:i + h] = x + y
            a[..., i + h:i + 2 * h] = x - y
        h *= 2
    return a


@pytest.mark.parametrize("b", [2, 4, 16, 128, 256])
def test_rotation_matches_butterfly(b):
    rng = np.random.default_rng(b)
    d = 4 * b
    U = rng.standard_normal((3, d))
    eps = Q.sign_mask(11, d)
    Y = Q.rotate_forward(U, eps, b)
    V = (U * eps).reshape(3, d // b, b)
    ref = _fwht_butterfly(V).reshape(3, d) / math.sqrt(b)
    assert np.max(np.abs(Y - ref)) < 1e-13


def test_b2_closed_form():
    U = np.array([[3.0, 1.0, -2.0, 5.0]])
    eps = Q.sign_mask(0, 4)
    v = U[0] * eps
    want = np.array([v[0] + v[1], v[0] - v[1], v[2] + v[3], v[2] - v[3]]) / math.sqrt(2)
    assert np.allclose(Q.rotate_forward(U, eps, 2)[0], want, rtol=0, atol=1e-15)


@pytest.mark.parametrize("b", [128, 256])
def test_rotation_orthogonal(b):
    d = 2 * b
    eps = Q.sign_mask(5, d)
    R = Q.rotate_forward(np.eye(d), eps, b).T          # column j = R e_j
    assert np.max(np.abs(R.T @ R - np.eye(d))) < 1e-14
    # block diagonal: nothing leaks between blocks
    assert np.all(R[:b, b:] == 0) and np.all(R[b:, :b] == 0)


def test_delta_input_is_flat():
    b, d = 128, 256
    eps = Q.sign_mask(9, d)
    H = scipy.linalg.hadamard(b)
    for j in (0, 5, 130):
        e = np.zeros((1, d))
        e[0, j] = 1.0
        y = Q.rotate_forward(e, eps, b)[0]
        blk = j // b
        assert np.allclose(np.abs(y[blk * b:(blk + 1) * b]), 1 / math.sqrt(b), atol=1e-16)
        assert np.array_equal(np.sign(y[blk * b:(blk + 1) * b]), eps[j] * H[:, j % b])
        other = np.delete(y, np.arange(blk * b, (blk + 1) * b))
        assert np.all(other == 0)


@pytest.mark.parametrize("b", [4, 128, 256])
def test_round_trip_and_isometry(b):
    rng = np.random.default_rng(100 + b)
    d = 3 * b
    U = rng.standard_normal((5, d))
    eps = Q.sign_mask(2, d)
    Y = Q.rotate_forward(U, eps, b)
    assert np.max(np.abs(Q.rotate_inverse(Y, eps, b) - U)) < 1e-13
    assert np.allclose(np.linalg.norm(Y, axis=1), np.linalg.norm(U, axis=1), rtol=1e-14)
