"""Polar coding baseline, fp64 definition (test infrastructure only).

The pages compare the joint 2D codebook with a polar code at the same rate:
amplitude and phase of each normalised pair quantised independently
(QAM-W, Methodology, Joint 2D Quantization; Experiments, the joint-versus-
polar ablation at about 4 bits per weight).  They give no design for the
polar code; the plainest one, used here:

  amplitude  Ka levels, the Lloyd-Max quantiser of the Rayleigh law (the
             amplitude of the unit circular Gaussian N(0, I_2)), computed
             from the law itself (closed-form cell moments), not sampled;
  phase      Kp uniform directions at angles 2 pi j / Kp, j = 0 .. Kp - 1;
  index      ia * Kp + ip, packed with B = ceil(log2(Ka Kp)) bits like the
             joint codec;
  decode     the point a_ia (cos phi_ip, sin phi_ip): a product table of
             Ka Kp entries that the joint decoder reads as its codebook.

Bit split: at 8 bits per pair (the ablation's rate) 8 amplitudes x 32 phases
has the least distortion of the power-of-two splits; at 11 bits 32 x 64; at 7
bits 8 x 16 (``tests/test_oracle_polar.py`` checks these orderings).

Decisions -- integers decided by floating point -- are made in fp32, the
precision of the GPU path, on z~ rounded to fp32:
  r  = sqrt(x*x + y*y), each operation rounded to fp32 (sqrt correctly rounded);
  ia = argmin_i |r - a_i| over the fp32 levels, ties to the lowest i;
  ip = argmax_j (x c_j + y s_j) over the fp32 directions (c_j, s_j), the
       nearest direction, ties to the lowest j.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf

from oracle import qamw_ref as O

SQRT_HALF_PI = math.sqrt(math.pi / 2.0)


# ---------------------------------------------------------------------------
# amplitude: Lloyd-Max on the Rayleigh law
# ---------------------------------------------------------------------------
def _rayleigh_mass(t):
    """P(R >= t) = exp(-t^2 / 2) for the Rayleigh law of |N(0, I_2)|."""
    t = np.asarray(t, dtype=np.float64)
    return np.where(np.isinf(t), 0.0, np.exp(-np.where(np.isinf(t), 0.0, t) ** 2 / 2.0))


def _rayleigh_first_moment(t):
    """int_0^t r * (r exp(-r^2/2)) dr = sqrt(pi/2) erf(t / sqrt 2) - t exp(-t^2/2)."""
    t = np.asarray(t, dtype=np.float64)
    finite = np.where(np.isinf(t), 0.0, t)
    val = SQRT_HALF_PI * erf(finite / math.sqrt(2.0)) - finite * np.exp(-finite ** 2 / 2.0)
    return np.where(np.isinf(t), SQRT_HALF_PI, val)


def rayleigh_cell_means(edges: np.ndarray) -> np.ndarray:
    """E[R | edges[i] <= R < edges[i+1]] for consecutive edges (edges[-1] may be inf)."""
    e = np.asarray(edges, dtype=np.float64)
    m1 = _rayleigh_first_moment(e)
    p = _rayleigh_mass(e)
    return (m1[1:] - m1[:-1]) / (p[:-1] - p[1:])


def rayleigh_lloyd_max(Ka: int, tol: float = 1e-12, max_iter: int = 200000):
    """Lloyd-Max levels (ascending, fp64) of a Ka-level quantiser of R ~ Rayleigh(1).

    Lloyd's two conditions, iterated to a fixed point: thresholds are the
    midpoints of adjacent levels, levels are the conditional means of their
    cells.  Starting levels: the Rayleigh quantiles at (i + 1/2) / Ka.  Stops
    when no level moves by more than ``tol`` (fp64 rounding keeps the last
    steps near 1e-13; the stored levels are fp32).  Returns (levels, iterations).
    """
    if Ka < 1:
        raise ValueError("Ka >= 1")
    q = (np.arange(Ka) + 0.5) / Ka
    a = np.sqrt(-2.0 * np.log1p(-q))
    for it in range(1, max_iter + 1):
        edges = np.concatenate([[0.0], 0.5 * (a[:-1] + a[1:]), [np.inf]])
        a_new = rayleigh_cell_means(edges)
        if np.max(np.abs(a_new - a)) <= tol:
            return a_new, it
        a = a_new
    return a, max_iter


# ---------------------------------------------------------------------------
# phase
# ---------------------------------------------------------------------------
def phase_directions(Kp: int) -> np.ndarray:
    """Unit vectors at angles 2 pi j / Kp, fp64 (Kp, 2)."""
    phi = 2.0 * np.pi * np.arange(Kp) / Kp
    return np.stack([np.cos(phi), np.sin(phi)], axis=1)


def product_table(levels: np.ndarray, dirs: np.ndarray) -> np.ndarray:
    """Decode table: entry ia * Kp + ip = a_ia * dir_ip, formed in fp64."""
    a = np.asarray(levels, dtype=np.float64)
    u = np.asarray(dirs, dtype=np.float64)
    return (a[:, None, None] * u[None, :, :]).reshape(-1, 2)


# ---------------------------------------------------------------------------
# quantiser
# ---------------------------------------------------------------------------
def polar_quantize(zt: np.ndarray, levels32: np.ndarray, dirs32: np.ndarray, chunk: int = 8192):
    """fp32 polar decision for points zt (M, 2): returns (ia, ip) int64.

    Exhaustive over the levels and the directions (definition in the module
    docstring); zt is rounded to fp32 first.
    """
    z = np.asarray(zt, dtype=np.float64).reshape(-1, 2).astype(np.float32)
    a = np.asarray(levels32, dtype=np.float32).reshape(-1)
    u = np.asarray(dirs32, dtype=np.float32).reshape(-1, 2)
    M = z.shape[0]
    ia = np.empty(M, dtype=np.int64)
    ip = np.empty(M, dtype=np.int64)
    for c0 in range(0, M, chunk):
        x, y = z[c0:c0 + chunk, 0], z[c0:c0 + chunk, 1]
        r = np.sqrt(x * x + y * y)                                       # fp32 ops
        ia[c0:c0 + chunk] = np.argmin(np.abs(r[:, None] - a[None, :]), axis=1)   # first minimum
        score = x[:, None] * u[None, :, 0] + y[:, None] * u[None, :, 1]  # fp32 ops
        ip[c0:c0 + chunk] = np.argmax(score, axis=1)                     # first maximum
    return ia, ip


def accept_polar(zt: np.ndarray, levels32, dirs32, ia_ref, ip_ref, ia_o, ip_o,
                 rel: float = O.NEAR_TIE_REL) -> np.ndarray:
    """Near-tie rule for another implementation's (ia, ip).

    A differing amplitude index is accepted when, in fp64, |r - a| of the
    other choice is within rel * r of the oracle's; a differing phase index
    when its inner product with z~ is within rel * r of the oracle's.
    """
    z = np.asarray(zt, dtype=np.float64).reshape(-1, 2)
    a = np.asarray(levels32, dtype=np.float32).astype(np.float64).reshape(-1)
    u = np.asarray(dirs32, dtype=np.float32).astype(np.float64).reshape(-1, 2)
    r = np.hypot(z[:, 0], z[:, 1])
    ia_ref = np.asarray(ia_ref).reshape(-1); ip_ref = np.asarray(ip_ref).reshape(-1)
    ia_o = np.asarray(ia_o).reshape(-1); ip_o = np.asarray(ip_o).reshape(-1)
    ok_range = (ia_o >= 0) & (ia_o < a.size) & (ip_o >= 0) & (ip_o < u.shape[0])
    ia_c = np.clip(ia_o, 0, a.size - 1)
    ip_c = np.clip(ip_o, 0, u.shape[0] - 1)
    tol = rel * r
    amp_ok = (ia_o == ia_ref) | (np.abs(np.abs(r - a[ia_c]) - np.abs(r - a[ia_ref])) < tol)
    s_ref = z[:, 0] * u[ip_ref, 0] + z[:, 1] * u[ip_ref, 1]
    s_o = z[:, 0] * u[ip_c, 0] + z[:, 1] * u[ip_c, 1]
    ph_ok = (ip_o == ip_ref) | (np.abs(s_ref - s_o) < tol)
    return ok_range & amp_ok & ph_ok


def encode_polar(W: np.ndarray, s: np.ndarray, sigma: np.ndarray, b: int, sign_seed: int,
                 levels32: np.ndarray, dirs32: np.ndarray, rows=None):
    """Encode rows of W with the polar code given the calibration (s, sigma).

    The transform (scale, row split, rotation, pairing, 1/sigma) is the joint
    codec's; only the per-pair quantiser differs.  Returns a dict with ia, ip,
    idx = ia * Kp + ip (M, d/2), packed (M, row_words), rho, rho_hat_bits, zt.
    """
    W = np.asarray(W)
    if rows is not None:
        W = W[np.asarray(rows)]
    Ka = np.asarray(levels32).size
    Kp = np.asarray(dirs32).reshape(-1, 2).shape[0]
    N, d = W.shape
    Zt, rho = O.normalized_pairs(W, s, sigma, b, sign_seed)
    ia, ip = polar_quantize(Zt.reshape(-1, 2), levels32, dirs32)
    ia = ia.reshape(N, d // 2)
    ip = ip.reshape(N, d // 2)
    idx = ia * Kp + ip
    return {
        "ia": ia, "ip": ip, "idx": idx,
        "packed": O.pack(idx, Ka * Kp, d),
        "rho": rho,
        "rho_hat_bits": O.to_f16_bits(rho),
        "zt": Zt,
    }
