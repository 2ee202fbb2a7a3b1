"""Pins of the polar-code oracle (oracle/polar.py) against closed forms,
independent numerical integration, brute force and the pages' ablation claim."""
import math
import os

import numpy as np
import pytest
from scipy import integrate, optimize

import workloads
from oracle import polar as P
from oracle import qamw_ref as O

CB_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "vector_codebook_codec_amd", "codebooks")


def rayleigh_pdf(r):
    return r * math.exp(-r * r / 2.0)


def quad_cell_mean(lo, hi):
    m1 = integrate.quad(lambda r: r * rayleigh_pdf(r), lo, hi, epsabs=1e-14, epsrel=1e-13, limit=200)[0]
    m0 = integrate.quad(rayleigh_pdf, lo, hi, epsabs=1e-14, epsrel=1e-13, limit=200)[0]
    return m1 / m0


def quad_distortion(levels):
    """E[(R - q(R))^2] for the nearest-level quantiser, by numerical integration."""
    a = np.sort(np.asarray(levels, dtype=np.float64))
    edges = np.concatenate([[0.0], 0.5 * (a[:-1] + a[1:]), [np.inf]])
    tot = 0.0
    for i, c in enumerate(a):
        tot += integrate.quad(lambda r: (r - c) ** 2 * rayleigh_pdf(r), edges[i], edges[i + 1],
                              epsabs=1e-14, epsrel=1e-12, limit=200)[0]
    return tot


def test_one_level_is_the_rayleigh_mean():
    a, _ = P.rayleigh_lloyd_max(1)
    assert a.shape == (1,)
    assert abs(a[0] - math.sqrt(math.pi / 2.0)) < 1e-14


@pytest.mark.parametrize("Ka", [2, 4, 8, 32])
def test_levels_meet_lloyd_conditions_by_quadrature(Ka):
    a, _ = P.rayleigh_lloyd_max(Ka)
    assert np.all(np.diff(a) > 0)
    edges = np.concatenate([[0.0], 0.5 * (a[:-1] + a[1:]), [np.inf]])
    for i in range(Ka):
        assert abs(quad_cell_mean(edges[i], edges[i + 1]) - a[i]) < 1e-9 * max(1.0, a[i])


@pytest.mark.parametrize("Ka", [2, 4])
def test_levels_are_a_local_minimum_of_the_distortion(Ka):
    a, _ = P.rayleigh_lloyd_max(Ka)
    d0 = quad_distortion(a)
    for i in range(Ka):
        for h in (-1e-3, 1e-3):
            b = a.copy()
            b[i] += h
            assert quad_distortion(b) > d0


def test_two_levels_match_brute_force_threshold_search():
    # one threshold t; each cell reconstructs at its conditional mean
    def dist(t):
        return quad_distortion([quad_cell_mean(0.0, t), quad_cell_mean(t, np.inf)])
    res = optimize.minimize_scalar(dist, bounds=(0.3, 3.0), method="bounded",
                                   options={"xatol": 1e-10})
    a, _ = P.rayleigh_lloyd_max(2)
    assert abs(0.5 * (a[0] + a[1]) - res.x) < 1e-5
    assert abs(dist(res.x) - quad_distortion(a)) < 1e-12


@pytest.mark.parametrize("Kp", [1, 2, 3, 8, 64])
def test_phase_directions(Kp):
    u = P.phase_directions(Kp)
    assert u.shape == (Kp, 2)
    assert np.allclose(np.hypot(u[:, 0], u[:, 1]), 1.0, atol=1e-15)
    ang = np.mod(np.arctan2(u[:, 1], u[:, 0]), 2 * np.pi)
    ref = 2 * np.pi * np.arange(Kp) / Kp
    diff = np.abs(np.angle(np.exp(1j * (ang - ref))))
    assert diff.max() < 1e-12


def brute_force_polar(z, levels, Kp):
    """fp64 geometric definition: nearest level to |z|, nearest angle 2 pi j / Kp."""
    r = np.hypot(z[:, 0], z[:, 1])
    dr = np.abs(r[:, None] - np.asarray(levels, np.float64)[None, :])
    ia = np.argmin(dr, axis=1)
    ang = np.arctan2(z[:, 1], z[:, 0])
    phi = 2 * np.pi * np.arange(Kp) / Kp
    dphi = np.abs(np.angle(np.exp(1j * (ang[:, None] - phi[None, :]))))
    ip = np.argmin(dphi, axis=1)
    part_r = np.sort(dr, axis=1)
    part_p = np.sort(dphi, axis=1)
    margin_r = part_r[:, 1] - part_r[:, 0] if dr.shape[1] > 1 else np.full(len(r), np.inf)
    margin_p = part_p[:, 1] - part_p[:, 0] if Kp > 1 else np.full(len(r), np.inf)
    return ia, ip, margin_r, margin_p


@pytest.mark.parametrize("Ka,Kp", [(8, 32), (32, 64), (4, 8), (1, 8), (4, 1), (16, 256)])
def test_quantize_matches_geometric_definition(Ka, Kp):
    a = P.rayleigh_lloyd_max(Ka)[0].astype(np.float32)
    u = P.phase_directions(Kp).astype(np.float32)
    z = np.random.default_rng(7 + Ka * 131 + Kp).standard_normal((40000, 2)) * 1.3
    ia, ip = P.polar_quantize(z, a, u)
    ia_b, ip_b, mr, mp = brute_force_polar(z.astype(np.float32).astype(np.float64), a, Kp)
    clear_r = mr > 1e-5
    clear_p = mp > 1e-5
    assert np.array_equal(ia[clear_r], ia_b[clear_r])
    assert np.array_equal(ip[clear_p], ip_b[clear_p])
    assert clear_r.mean() > 0.99 and clear_p.mean() > 0.99


def test_quantize_special_cases():
    a = P.rayleigh_lloyd_max(8)[0].astype(np.float32)
    u = P.phase_directions(32).astype(np.float32)
    # the origin: every distance to the first level is smallest, every score 0
    ia, ip = P.polar_quantize(np.zeros((3, 2)), a, u)
    assert ia.tolist() == [0, 0, 0] and ip.tolist() == [0, 0, 0]
    # points on the table itself decode to themselves
    pts = P.product_table(a.astype(np.float64), u.astype(np.float64))
    ia, ip = P.polar_quantize(pts, a, u)
    assert np.array_equal(ia * 32 + ip, np.arange(8 * 32))
    # one direction: every phase index is 0; one level: every amplitude index is 0
    z = np.random.default_rng(3).standard_normal((1000, 2))
    assert not P.polar_quantize(z, a, P.phase_directions(1).astype(np.float32))[1].any()
    assert not P.polar_quantize(z, np.array([1.25], np.float32), u)[0].any()
    # two directions: the sign of x decides
    ia, ip = P.polar_quantize(np.array([[2.0, 0.3], [-2.0, 0.3], [-1e-3, -5.0]]), a,
                              P.phase_directions(2).astype(np.float32))
    assert ip.tolist() == [0, 1, 1]


def polar_distortion(z, Ka, Kp):
    a = P.rayleigh_lloyd_max(Ka)[0]
    u = P.phase_directions(Kp)
    ia, ip = P.polar_quantize(z, a.astype(np.float32), u.astype(np.float32))
    zh = P.product_table(a, u)[ia * Kp + ip]
    return float(np.mean(np.sum((z - zh) ** 2, axis=1)))


def test_bit_splits_and_the_joint_versus_polar_claim():
    # fresh samples (seed 11), not the codebook's training draw (seed 1)
    z = workloads.gaussian_samples(1 << 17, 11)
    d8 = {ka: polar_distortion(z, ka, 256 // ka) for ka in (4, 8, 16)}
    assert d8[8] < d8[4] and d8[8] < d8[16]
    d7 = {ka: polar_distortion(z, ka, 128 // ka) for ka in (4, 8, 16)}
    assert d7[8] < d7[4] and d7[8] < d7[16]
    d11 = {ka: polar_distortion(z, ka, 2048 // ka) for ka in (16, 32, 64)}
    assert d11[32] < d11[16] and d11[32] < d11[64]
    # the pages' ablation rate (~4 bits per weight, 8 bits per pair): the
    # joint 2D codebook has less distortion than the polar code
    C = np.fromfile(os.path.join(CB_DIR, "qamw_K256.f32"), dtype="<f4").reshape(-1, 2)
    idx, dmin = __import__("oracle.lloyd", fromlist=["assign"]).assign(z, C.astype(np.float64))
    assert float(dmin.mean()) < d8[8]


@pytest.mark.parametrize("Ka,Kp", [(8, 16), (8, 32), (32, 64), (16, 256), (1, 8), (2, 2), (4, 1), (4, 8)])
def test_stored_tables(Ka, Kp):
    base = os.path.join(CB_DIR, f"polar_A{Ka}_P{Kp}")
    lv = np.fromfile(base + "_levels.f32", dtype="<f4")
    dr = np.fromfile(base + "_dirs.f32", dtype="<f4").reshape(-1, 2)
    tb = np.fromfile(base + ".f32", dtype="<f4").reshape(-1, 2)
    assert lv.shape == (Ka,) and dr.shape == (Kp, 2) and tb.shape == (Ka * Kp, 2)
    a = P.rayleigh_lloyd_max(Ka)[0]
    assert np.array_equal(lv, a.astype(np.float32))
    assert np.all(np.abs(np.hypot(dr[:, 0].astype(np.float64), dr[:, 1]) - 1.0) < 1e-7)
    prod = lv.astype(np.float64)[:, None, None] * dr.astype(np.float64)[None, :, :]
    assert np.allclose(tb, prod.reshape(-1, 2), rtol=3e-7, atol=1e-7)


def test_accept_polar_rejects_a_planted_mistake():
    a = P.rayleigh_lloyd_max(8)[0].astype(np.float32)
    u = P.phase_directions(32).astype(np.float32)
    z = np.random.default_rng(5).standard_normal((5000, 2))
    ia, ip = P.polar_quantize(z, a, u)
    assert P.accept_polar(z, a, u, ia, ip, ia, ip).all()
    bad_ia = ia.copy(); bad_ia[17] = (bad_ia[17] + 3) % 8
    bad_ip = ip.copy(); bad_ip[23] = (bad_ip[23] + 5) % 32
    ok = P.accept_polar(z, a, u, ia, ip, bad_ia, bad_ip)
    assert not ok[17] and not ok[23] and ok.sum() == len(z) - 2
    assert not P.accept_polar(z[:1], a, u, ia[:1], ip[:1], np.array([8]), ip[:1]).any()


def test_encode_polar_round_trip():
    wl = workloads.get("c1_256x512")
    Wf = wl.W_f32()
    s, sigma, _ = O.calibrate(Wf, wl.r, wl.alpha, wl.block, wl.sign_seed)
    Ka, Kp = 8, 32
    a = P.rayleigh_lloyd_max(Ka)[0]
    u = P.phase_directions(Kp)
    enc = P.encode_polar(Wf, s, sigma, wl.block, wl.sign_seed, a.astype(np.float32), u.astype(np.float32))
    idx = O.unpack(enc["packed"], Ka * Kp, wl.d)
    assert np.array_equal(idx, enc["ia"] * Kp + enc["ip"])
    table = P.product_table(a, u).astype(np.float32)
    # the quantiser's own error on z~ equals the decoded matrix's in the rotated domain
    zt = enc["zt"].reshape(-1, 2)
    zh = table.astype(np.float64)[idx.reshape(-1)]
    dz = float(np.mean(np.sum((zt - zh) ** 2, axis=1)))
    assert 0.5 * polar_distortion(workloads.gaussian_samples(1 << 15, 12), Ka, Kp) < dz < 2.0 * 0.019
    Wh = O.decode(enc["packed"], enc["rho_hat_bits"], s, sigma, wl.block, wl.sign_seed, table, wl.d)
    rel = np.linalg.norm(Wh - Wf) / np.linalg.norm(Wf)
    assert 0.05 < rel < 0.2
