"""Pins for the oracle's encode/decode steps (CPU only).

Each test checks the oracle against something other than itself: closed
forms (alpha = 0 and 1, constant-amplitude rows, quadrant cells), the
Rayleigh mean, brute force written here in plain Python, exact arithmetic
under power-of-two scaling, hand-computed packed words, and a lossless
codebook that must reproduce its input.
"""
import json
import math
import os

import numpy as np
import pytest

from conftest import GOLDEN
from oracle import qamw_ref as Q


# ---------------------------------------------------------------- scaling / norm
def test_activation_scale_closed_forms():
    r = np.random.default_rng(0).lognormal(0, 1, 64).astype(np.float32)
    assert np.all(Q.activation_scale(r, 0.0) == 1.0)
    assert np.array_equal(Q.activation_scale(r, 1.0), r.astype(np.float64))
    assert np.allclose(Q.activation_scale(r, 0.5), np.sqrt(r.astype(np.float64)), rtol=1e-15)


def test_row_split_unit_rows_and_zero_row():
    W = np.random.default_rng(1).standard_normal((6, 40))
    W[3] = 0.0
    rho, U = Q.row_split(W)
    assert rho[3] == 0.0 and np.all(U[3] == 0.0)
    keep = np.arange(6) != 3
    assert np.allclose(np.linalg.norm(U[keep], axis=1), 1.0, atol=1e-15)
    assert np.allclose(rho[keep], np.linalg.norm(W[keep], axis=1), rtol=1e-15)


def test_power_of_two_equivariance():
    """W -> 2^k W scales rho by 2^k exactly and changes neither sigma nor indices."""
    rng = np.random.default_rng(2)
    W = rng.standard_normal((32, 64)).astype(np.float32) * 0.02
    r = rng.lognormal(0, 0.5, 64).astype(np.float32)
    C = np.random.default_rng(3).standard_normal((16, 2)).astype(np.float32)
    s, sig, rho = Q.calibrate(W, r, 0.5, 16, 4)
    e = Q.encode(W, s, sig, 16, 4, C)
    for k in (-7, 5):
        s2, sig2, rho2 = Q.calibrate(W * 2.0 ** k, r, 0.5, 16, 4)
        assert np.array_equal(rho2, rho * 2.0 ** k)
        assert np.array_equal(sig2, sig)
        e2 = Q.encode(W * 2.0 ** k, s2, sig2, 16, 4, C)
        assert np.array_equal(e2["idx"], e["idx"])


# ---------------------------------------------------------------- sigma
def test_sigma_constant_amplitude_closed_form():
    """Rows whose rotated pairs all have the same amplitude a: after the row
    split every pair has amplitude 1/sqrt(d/2), so sigma = that / sqrt(pi/2)."""
    rng = np.random.default_rng(4)
    N, d, b, seed = 16, 256, 128, 6
    phase = rng.uniform(0, 2 * np.pi, (N, d // 2))
    a = 0.37
    Y = np.empty((N, d))
    Y[:, 0::2] = a * np.cos(phase)
    Y[:, 1::2] = a * np.sin(phase)
    W = Q.rotate_inverse(Y, Q.sign_mask(seed, d), b)
    _, sig, _ = Q.calibrate(W, np.ones(d), 0.0, b, seed)
    want = (1.0 / math.sqrt(d / 2)) / math.sqrt(math.pi / 2)
    assert np.allclose(sig, want, rtol=1e-12)


def test_sigma_rayleigh_mean():
    """For i.i.d. N(0, s^2 I_2) pairs the estimator is unbiased with relative
    standard deviation sqrt(4/pi - 1) / sqrt(N) = 0.5227 / sqrt(N)."""
    rng = np.random.default_rng(5)
    N, P, sd = 20000, 8, 0.3
    Z = rng.standard_normal((N, P, 2)) * sd
    sig = Q.sigma_from_pairs(Z)
    rel_sd = math.sqrt(4 / math.pi - 1) / math.sqrt(N)
    assert abs(math.sqrt(4 / math.pi - 1) - 0.5227) < 1e-4
    assert np.all(np.abs(sig / sd - 1) < 5 * rel_sd)


def test_sigma_gaussian_rows():
    """Normalised Gaussian rows are uniform on the sphere; rotated pairs are then
    close to circular Gaussian with per-component deviation 1/sqrt(d)."""
    W = np.random.default_rng(6).standard_normal((4096, 512))
    _, sig, _ = Q.calibrate(W, np.ones(512), 0.5, 128, 0)
    assert np.all(np.abs(sig * math.sqrt(512) - 1) < 6 * 0.5227 / math.sqrt(4096))


# ---------------------------------------------------------------- nearest centroid
def _brute_force_f32(z, C):
    """Plain loop: first centroid with the smallest fp32 squared distance."""
    best, bi = None, -1
    zx, zy = np.float32(z[0]), np.float32(z[1])
    for i, (cx, cy) in enumerate(C):
        dx = zx - np.float32(cx)
        dy = zy - np.float32(cy)
        dd = np.float32(dx * dx) + np.float32(dy * dy)
        if best is None or dd < best:
            best, bi = dd, i
    return bi


def test_argmin_brute_force():
    rng = np.random.default_rng(7)
    C = rng.standard_normal((37, 2)).astype(np.float32)
    Z = rng.standard_normal((300, 2)) * 1.3
    idx, d_at, d_best, _ = Q.nearest_centroid(Z, C)
    want = [_brute_force_f32(z, C) for z in Z]
    assert np.array_equal(idx, want)
    assert np.all(d_at - d_best <= 1e-6 * (Z ** 2).sum(1))


def test_argmin_quadrant_closed_form():
    C = np.array([[1, 1], [-1, 1], [-1, -1], [1, -1]], dtype=np.float32)
    Z = np.random.default_rng(8).standard_normal((1000, 2))
    Z = Z[np.min(np.abs(Z), axis=1) > 1e-3]
    idx, *_ = Q.nearest_centroid(Z, C)
    quad = np.where(Z[:, 0] > 0, np.where(Z[:, 1] > 0, 0, 3), np.where(Z[:, 1] > 0, 1, 2))
    assert np.array_equal(idx, quad)


def test_argmin_exact_ties_lowest_index():
    C = np.array([[1, 0], [0, 1], [-1, 0], [0, -1]], dtype=np.float32)
    idx, *_ = Q.nearest_centroid(np.array([[0.0, 0.0]]), C)
    assert idx[0] == 0
    idx, *_ = Q.nearest_centroid(np.array([[-0.5, 0.5]]), C)
    assert idx[0] == 1                       # tie between 1 and 2
    C2 = np.array([[1, 1], [0, 0], [1, 1]], dtype=np.float32)
    idx, *_ = Q.nearest_centroid(np.array([[0.5, 0.5], [2.0, 2.0]]), C2)
    assert list(idx) == [0, 0]               # duplicates and a two-way tie


def test_argmin_single_centroid():
    idx, *_ = Q.nearest_centroid(np.random.default_rng(9).standard_normal((5, 2)),
                                 np.array([[0.3, -0.2]], dtype=np.float32))
    assert np.all(idx == 0)


def test_accept_index_rule():
    C = np.array([[0, 0], [1, 0], [0.5, 10]], dtype=np.float32)
    z = np.array([[0.5, 0.0], [0.2, 0.0]])
    ref = np.array([0, 0])
    # z0 is equidistant from 0 and 1: accepted; z1 is not a tie: rejected
    assert list(Q.accept_index(z, C, ref, np.array([1, 1]))) == [True, False]
    assert list(Q.accept_index(z, C, ref, np.array([0, 0]))) == [True, True]
    assert list(Q.accept_index(z, C, ref, np.array([7, 2]))) == [False, False]


# ---------------------------------------------------------------- packing
def test_packed_row_words_values():
    assert Q.index_bits(2) == 1 and Q.index_bits(256) == 8
    assert Q.index_bits(2048) == 11 and Q.index_bits(4096) == 12 and Q.index_bits(3) == 2
    assert Q.packed_row_words(11008, 2048) == 1892
    assert Q.packed_row_words(4096, 2048) == 704
    assert Q.packed_row_words(512, 256) == 64
    assert Q.packed_row_words(13824, 4096) == 2592
    assert Q.packed_row_words(13824, 1024) == 2160
    assert Q.packed_row_words(12, 2048) == 4


def test_pack_hand_words():
    with open(os.path.join(GOLDEN, "pack_hand_words.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        assert Q.index_bits(c["K"]) == c["B"]
        words = Q.pack(np.array([c["idx"]]), c["K"], c["d"])[0]
        assert [int(w) for w in words] == [int(w, 16) for w in c["words"]], c["why"]
        assert list(Q.unpack(words[None, :], c["K"], c["d"])[0]) == c["idx"]


@pytest.mark.parametrize("B", list(range(1, 13)))
def test_pack_round_trip(B):
    K = 1 << B
    rng = np.random.default_rng(B)
    for d in (2, 34, 64, 250, 512):
        idx = rng.integers(0, K, size=(3, d // 2))
        packed = Q.pack(idx, K, d)
        assert packed.shape == (3, Q.packed_row_words(d, K))
        assert np.array_equal(Q.unpack(packed, K, d), idx)
        # padding bits after the last index are zero
        total = (d // 2) * B
        stream = np.unpackbits(packed.astype("<u4").view(np.uint8), axis=1, bitorder="little")
        assert not stream[:, total:].any()


# ---------------------------------------------------------------- end to end
def test_lossless_codebook_round_trip():
    """With the codebook equal to the set of normalised pairs, every pair is
    coded at distance 0 and decode returns W * rho_hat / rho.  This pins the
    order, signs, pairing and every inverse of the pipeline."""
    rng = np.random.default_rng(10)
    N, d, b, seed = 4, 8, 4, 3
    W = rng.standard_normal((N, d))
    r = rng.lognormal(0, 0.5, d)
    s, sig, rho = Q.calibrate(W, r, 0.5, b, seed)
    Zt, _ = Q.normalized_pairs(W, s, sig, b, seed)
    C = Zt.reshape(-1, 2).astype(np.float32)
    e = Q.encode(W, s, sig, b, seed, C)
    assert np.all(e["d64_best"] < 1e-12)
    assert np.array_equal(e["idx"].reshape(-1), np.arange(N * d // 2))
    Wh = Q.decode(e["packed"], e["rho_hat_bits"], s, sig, b, seed, C, d)
    rho_hat = Q.f16_bits_to_f64(e["rho_hat_bits"])
    want = W * (rho_hat / rho)[:, None]
    assert np.max(np.abs(Wh - want)) < 1e-6 * np.max(np.abs(want))
    # without s decode returns W' = W diag(s)
    Wp = Q.decode(e["packed"], e["rho_hat_bits"], None, sig, b, seed, C, d)
    want = W * s[None, :] * (rho_hat / rho)[:, None]
    assert np.max(np.abs(Wp - want)) < 1e-6 * np.max(np.abs(want))


def test_exact_round_trip_before_quantization():
    rng = np.random.default_rng(11)
    W = rng.standard_normal((5, 512)) * 0.02
    r = rng.lognormal(0, 1, 512)
    s, sig, rho = Q.calibrate(W, r, 0.5, 128, 0)
    Zt, _ = Q.normalized_pairs(W, s, sig, 128, 0)
    Y = (Zt * sig[None, :, None]).reshape(5, 512)
    back = rho[:, None] * Q.rotate_inverse(Y, Q.sign_mask(0, 512), 128) / s[None, :]
    assert np.max(np.abs(back - W)) < 1e-15


def test_degenerate_rows_and_columns():
    rng = np.random.default_rng(12)
    N, d, b = 6, 32, 8
    W = rng.standard_normal((N, d))
    W[2] = 0.0
    C = rng.standard_normal((8, 2)).astype(np.float32)
    s = np.ones(d)
    sig = np.abs(rng.standard_normal(d // 2)) + 0.1
    sig[5] = 0.0
    e = Q.encode(W, s, sig, b, 1, C)
    # a zero row has rho 0 and decodes to exact zeros
    assert e["rho"][2] == 0.0 and e["rho_hat_bits"][2] == 0
    # sigma_k = 0: z~ := 0 -> nearest centroid of the origin
    origin, *_ = Q.nearest_centroid(np.zeros((1, 2)), C)
    assert np.all(e["idx"][:, 5] == origin[0])
    Wh = Q.decode(e["packed"], e["rho_hat_bits"], s, sig, b, 1, C, d)
    assert np.all(Wh[2] == 0.0)
    # indices >= K in a hand-made stream are clamped to K - 1 (B = 3 allows 8 > K = 5)
    K = 5
    idx = np.full((1, d // 2), 7)
    Wc = Q.decode(Q.pack(idx, K, d), np.array([0x3C00], np.uint16), None, np.ones(d // 2), b, 1,
                  C[:K], d)
    Wk = Q.decode(Q.pack(np.full((1, d // 2), K - 1), K, d), np.array([0x3C00], np.uint16), None,
                  np.ones(d // 2), b, 1, C[:K], d)
    assert np.array_equal(Wc, Wk)


def test_dead_channel_decodes_as_zero():
    """r_j = 0 (a channel whose activations are all zero) gives s_j = 0 for
    alpha > 0: the channel is zeroed before quantisation, decodes as 0 instead
    of dividing by zero, and its activations are dropped by the rotated-form
    product, so X W^^T equals X~ W'^T on the other channels.  Pinned
    independently of inverse_scale: the lossless codebook reproduces every
    other column exactly up to rho_hat / rho, and the product is checked
    against a plain matmul with column j removed."""
    rng = np.random.default_rng(13)
    N, d, b, seed, j = 4, 16, 8, 2, 5
    W = rng.standard_normal((N, d))
    r = rng.lognormal(0, 0.5, d)
    r[j] = 0.0
    s, sig, rho = Q.calibrate(W, r, 0.5, b, seed)
    assert s[j] == 0.0 and np.all(np.isfinite(sig))
    Zt, _ = Q.normalized_pairs(W, s, sig, b, seed)
    C = Zt.reshape(-1, 2).astype(np.float32)
    e = Q.encode(W, s, sig, b, seed, C)
    Wh = Q.decode(e["packed"], e["rho_hat_bits"], s, sig, b, seed, C, d)
    assert np.all(np.isfinite(Wh)) and np.all(Wh[:, j] == 0.0)
    rho_hat = Q.f16_bits_to_f64(e["rho_hat_bits"])
    keep = np.arange(d) != j
    want = W * (rho_hat / rho)[:, None]
    assert np.max(np.abs(Wh[:, keep] - want[:, keep])) < 1e-5 * np.max(np.abs(want))
    X = rng.standard_normal((3, d))
    Xr = Q.rotate_activations(X, s, b, seed)
    assert np.all(np.isfinite(Xr))
    Y = Q.decode_matmul(X, e["packed"], e["rho_hat_bits"], s, sig, b, seed, C, d)
    assert np.allclose(Y, X[:, keep] @ Wh[:, keep].T, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- fp16 / bf16 rounding
def test_half_rounding_pins():
    one = 1.0
    f16 = lambda x: float(Q.f16_bits_to_f64(Q.to_f16_bits(np.array([x])))[0])
    bf = lambda x: float(Q.bf16_bits_to_f64(Q.to_bf16_bits(np.array([x])))[0])
    assert f16(one + 2 ** -11) == 1.0                      # tie -> even
    assert f16(one + 3 * 2 ** -11) == 1.0 + 2 ** -9        # tie -> even (up)
    assert f16(one + 2 ** -11 + 2 ** -40) == 1.0 + 2 ** -10
    assert bf(one + 2 ** -8) == 1.0
    assert bf(one + 3 * 2 ** -8) == 1.0 + 2 ** -6
    # one rounding straight from fp64 (a detour through fp32 would land on 1.0)
    assert bf(one + 2 ** -8 + 2 ** -30) == 1.0 + 2 ** -7
    assert bf(-0.15625) == -0.15625 and bf(0.0) == 0.0
    assert Q.to_bf16_bits(np.array([1.0]))[0] == 0x3F80
    assert Q.to_f16_bits(np.array([1.0]))[0] == 0x3C00


# ---------------------------------------------------------------- layer-output error
def test_trace_identity():
    rng = np.random.default_rng(13)
    X = rng.standard_normal((64, 16))
    dW = rng.standard_normal((8, 16))
    a = Q.output_error_direct(X, dW)
    t = Q.output_error_trace(X, dW)
    assert abs(a - t) <= 1e-12 * abs(a)


def test_output_weighted_error_is_diagonal_trace():
    """With orthogonal activation columns, X^T X = n diag(r^2) and the trace form
    reduces to n * sum_j r_j^2 ||dW[:, j]||^2."""
    rng = np.random.default_rng(14)
    n, d = 64, 16
    Qm, _ = np.linalg.qr(rng.standard_normal((n, d)))
    r = rng.lognormal(0, 1, d)
    X = Qm * (math.sqrt(n) * r)[None, :]
    dW = rng.standard_normal((8, d))
    assert abs(Q.output_error_trace(X, dW) - n * Q.output_weighted_error(r, dW)) < 1e-10 * Q.output_error_trace(X, dW)
