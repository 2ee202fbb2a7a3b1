"""QAM-W codec, fp64 definition (test infrastructure only).

Pipeline, per weight row (QAM-W, Methodology: The QAM-W Codec):

  activation-aware scaling   W'[n, j] = W[n, j] * s_j,  s_j = r_j ** alpha
  scale/direction split      rho_n = ||W'_n||_2,  u_n = W'_n / rho_n
  rotation                   y_n = R_fwd u_n, R_fwd = (I (x) H_b / sqrt(b)) diag(eps)
  pairing                    z_{n,k} = (y_{n,2k}, y_{n,2k+1})
  calibration                sigma_k = mean_n |z_{n,k}| / sqrt(pi/2)
  joint 2D quantisation      idx_{n,k} = nearest centroid of z_{n,k} / sigma_k
  packing                    B = ceil(log2 K) bits per index, LSB-first stream
  decode                     unpack -> C[idx] * sigma_k -> R_fwd^T -> * rho_hat_n / s_j

Readings of points the pages leave open (sign generator, Hadamard order,
sigma estimator, bit layout, tie rule, metadata precision) are stated at the
function that takes them.
"""
from __future__ import annotations

import math

import numpy as np

MASK64 = (1 << 64) - 1
SPLITMIX64_GAMMA = 0x9E3779B97F4A7C15
NEAR_TIE_REL = 1e-6
SQRT_HALF_PI = math.sqrt(math.pi / 2.0)


# ---------------------------------------------------------------------------
# sign mask
# ---------------------------------------------------------------------------
def splitmix64(seed: int, count: int) -> list:
    """First ``count`` outputs of SplitMix64 (Steele, Lea & Flood, OOPSLA 2014)
    seeded with ``seed``, as Python ints.

    Stateful form: add the golden-gamma increment to the state, then apply the
    variant-13 finaliser (xor-shift 30, multiply, xor-shift 27, multiply,
    xor-shift 31).
    """
    out = []
    state = seed & MASK64
    for _ in range(count):
        state = (state + SPLITMIX64_GAMMA) & MASK64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
        out.append(z ^ (z >> 31))
    return out


def sign_mask(seed: int, d: int) -> np.ndarray:
    """eps_j in {+1, -1}, j = 0..d-1, fp64.

    The rotation is deterministic and sign-masked (QAM-W, Methodology,
    Deterministic Rotation) but the pages do not say how the signs are drawn.
    Reading: eps_j = -1 exactly when bit 63 of the j-th SplitMix64 output for
    ``seed`` is set.  One mask serves every row of a matrix.
    """
    return np.array([-1.0 if (v >> 63) else 1.0 for v in splitmix64(seed, d)],
                    dtype=np.float64)


# ---------------------------------------------------------------------------
# rotation
# ---------------------------------------------------------------------------
def _popcount(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.int64)
    c = np.zeros_like(x)
    for t in range(20):
        c += (x >> t) & 1
    return c


def sylvester_hadamard(b: int) -> np.ndarray:
    """Sylvester-order Hadamard matrix H[i, k] = (-1) ** popcount(i & k), fp64."""
    if b < 1 or (b & (b - 1)):
        raise ValueError("block size must be a power of two")
    i = np.arange(b)
    return np.where(_popcount(i[:, None] & i[None, :]) % 2 == 0, 1.0, -1.0)


def rotate_forward(U: np.ndarray, eps: np.ndarray, b: int) -> np.ndarray:
    """y = R_fwd u for every row: signs first, then an orthonormal Hadamard
    transform on each contiguous block [beta*b, beta*b + b) of the row
    (QAM-W, Methodology, Deterministic Rotation).

    Reading: R_fwd = (I (x) H_b / sqrt(b)) diag(eps), Sylvester order, d % b == 0.
    Computed densely, one b x b product per block.
    """
    U = np.asarray(U, dtype=np.float64)
    N, d = U.shape
    if d % b:
        raise ValueError("row length must be a multiple of the block size")
    H = sylvester_hadamard(b)
    V = (U * eps[None, :]).reshape(N, d // b, b)
    Y = V @ H.T / math.sqrt(b)
    return Y.reshape(N, d)


def rotate_inverse(Y: np.ndarray, eps: np.ndarray, b: int) -> np.ndarray:
    """u = R_fwd^T y = diag(eps) (I (x) H_b / sqrt(b)) y (H_b is symmetric)."""
    Y = np.asarray(Y, dtype=np.float64)
    N, d = Y.shape
    H = sylvester_hadamard(b)
    V = (Y.reshape(N, d // b, b) @ H.T / math.sqrt(b)).reshape(N, d)
    return V * eps[None, :]


# ---------------------------------------------------------------------------
# encode steps
# ---------------------------------------------------------------------------
def activation_scale(r: np.ndarray, alpha: float) -> np.ndarray:
    """s_j = r_j ** alpha (QAM-W, Methodology, Activation-Aware Scaling).

    The pages give s_j only up to proportionality; reading: constant 1, so
    alpha = 0 gives s = 1 exactly.  Direction: the codec quantises W diag(s)
    and decode divides by s_j again.
    """
    return np.asarray(r, dtype=np.float64) ** float(alpha)


def row_split(Wp: np.ndarray):
    """rho_n = ||W'_n||_2 and u_n = W'_n / rho_n (u_n = 0 when rho_n = 0)
    (QAM-W, Methodology, Separation of Scale and Direction)."""
    Wp = np.asarray(Wp, dtype=np.float64)
    rho = np.sqrt(np.sum(Wp * Wp, axis=1))
    safe = np.where(rho > 0.0, rho, 1.0)
    U = np.where(rho[:, None] > 0.0, Wp / safe[:, None], 0.0)
    return rho, U


def pairs(Y: np.ndarray) -> np.ndarray:
    """z_{n,k} = (y_{n,2k}, y_{n,2k+1}) -> array (N, d/2, 2)
    (QAM-W, Methodology, Pairing and Calibration)."""
    Y = np.asarray(Y)
    N, d = Y.shape
    return Y.reshape(N, d // 2, 2)


def sigma_from_pairs(Z: np.ndarray) -> np.ndarray:
    """sigma_k from the mean pair amplitude over rows, under a circular
    Gaussian model (QAM-W, Methodology, Pairing and Calibration).

    Reading: for a circular Gaussian with per-component deviation sigma the
    amplitude is Rayleigh with mean sigma * sqrt(pi/2), so
    sigma_k = mean_n |z_{n,k}| / sqrt(pi/2).
    """
    amp = np.hypot(Z[:, :, 0], Z[:, :, 1])
    return amp.sum(axis=0) / (Z.shape[0] * SQRT_HALF_PI)


def calibrate(W: np.ndarray, r: np.ndarray, alpha: float, b: int, sign_seed: int):
    """Calibration pass over the whole matrix: returns (s, sigma, rho), fp64."""
    W = np.asarray(W, dtype=np.float64)
    s = activation_scale(r, alpha)
    rho, U = row_split(W * s[None, :])
    Y = rotate_forward(U, sign_mask(sign_seed, W.shape[1]), b)
    return s, sigma_from_pairs(pairs(Y)), rho


def normalized_pairs(W: np.ndarray, s: np.ndarray, sigma: np.ndarray, b: int,
                     sign_seed: int):
    """z~_{n,k} = z_{n,k} / sigma_k (0 where sigma_k = 0), together with rho.

    Returns (Zt (N, d/2, 2) fp64, rho (N,) fp64).
    """
    W = np.asarray(W, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    sigma = np.asarray(sigma, dtype=np.float64)
    rho, U = row_split(W * s[None, :])
    Z = pairs(rotate_forward(U, sign_mask(sign_seed, W.shape[1]), b))
    safe = np.where(sigma > 0.0, sigma, 1.0)
    Zt = np.where(sigma[None, :, None] > 0.0, Z / safe[None, :, None], 0.0)
    return Zt, rho


def nearest_centroid(zt: np.ndarray, C: np.ndarray):
    """Nearest centroid of each 2D point (QAM-W, Methodology, Joint 2D
    Quantization): argmin_c |z~ - C_c|^2, exhaustive over the codebook.

    The pages fix no arithmetic precision.  The index -- an integer decided by
    floating point -- is decided in fp32, the precision of the GPU path: z~ is
    rounded to fp32 and the squared distances are formed in fp32 with the
    codebook's fp32 values.  Exact ties go to the lowest index (reading).
    The fp64 distances are returned alongside for near-tie accounting.

    zt: (M, 2) fp64; C: (K, 2) fp32.
    Returns (idx int64 (M,), d64_at_idx (M,), d64_best (M,), d64_second (M,)).
    """
    zt = np.asarray(zt, dtype=np.float64).reshape(-1, 2)
    C32 = np.asarray(C, dtype=np.float32).reshape(-1, 2)
    C64 = C32.astype(np.float64)
    z32 = zt.astype(np.float32)
    dx32 = z32[:, 0:1] - C32[None, :, 0]
    dy32 = z32[:, 1:2] - C32[None, :, 1]
    D32 = dx32 * dx32 + dy32 * dy32
    idx = np.argmin(D32, axis=1)
    D64 = (zt[:, 0:1] - C64[None, :, 0]) ** 2 + (zt[:, 1:2] - C64[None, :, 1]) ** 2
    rows = np.arange(zt.shape[0])
    if C64.shape[0] >= 2:
        part = np.partition(D64, 1, axis=1)
        best, second = part[:, 0], part[:, 1]
    else:
        best, second = D64[:, 0], np.full(zt.shape[0], np.inf)
    return idx.astype(np.int64), D64[rows, idx], best, second


def accept_index(zt: np.ndarray, C: np.ndarray, idx_ref: np.ndarray,
                 idx_other: np.ndarray, rel: float = NEAR_TIE_REL) -> np.ndarray:
    """Near-tie rule for comparing another implementation's indices.

    An index differing from the oracle's is accepted only when its fp64
    squared distance is within rel * |z~|^2 of the oracle choice's.  Returns
    a boolean array: True where the indices agree or the pair is a near-tie.
    """
    zt = np.asarray(zt, dtype=np.float64).reshape(-1, 2)
    C64 = np.asarray(C, dtype=np.float32).astype(np.float64).reshape(-1, 2)
    a = np.asarray(idx_ref).reshape(-1)
    o = np.asarray(idx_other).reshape(-1)
    oc = np.clip(o, 0, C64.shape[0] - 1)
    da = ((zt - C64[a]) ** 2).sum(axis=1)
    do = ((zt - C64[oc]) ** 2).sum(axis=1)
    tol = rel * (zt ** 2).sum(axis=1)
    return (a == o) | ((o < C64.shape[0]) & (np.abs(do - da) < tol))


# ---------------------------------------------------------------------------
# bit packing
# ---------------------------------------------------------------------------
def index_bits(K: int) -> int:
    """B = ceil(log2 K) bits per index (K >= 2); K = 1 needs none."""
    return (int(K) - 1).bit_length()


def packed_row_words(d: int, K: int) -> int:
    """uint32 words per packed row: ceil((d/2) * B / 32), rounded up to a
    multiple of 4 so that every row starts on a 16-byte boundary."""
    bits = (d // 2) * index_bits(K)
    words = -(-bits // 32)
    return -(-words // 4) * 4


def pack(idx: np.ndarray, K: int, d: int) -> np.ndarray:
    """Pack indices (N, d/2) into (N, row_words) uint32.

    The decoder unpacks indices (QAM-W, Methodology, Decoding); the layout is
    not given.  Reading: each row is an LSB-first bitstream -- bit t of the
    stream is bit (t mod 32) of word t // 32 -- and index k occupies stream
    bits [k*B, k*B + B), least significant bit first.  Padding bits are 0.
    """
    idx = np.asarray(idx, dtype=np.int64)
    N, P = idx.shape
    B = index_bits(K)
    rw = packed_row_words(d, K)
    if B == 0:
        return np.zeros((N, rw), dtype=np.uint32)
    if (idx < 0).any() or (idx >= (1 << B)).any():
        raise ValueError("index out of range for the bit width")
    bits = (idx[:, :, None] >> np.arange(B)[None, None, :]) & 1        # (N, P, B)
    stream = np.zeros((N, rw * 32), dtype=np.uint64)
    stream[:, : P * B] = bits.reshape(N, P * B)
    weights = np.uint64(1) << np.arange(32, dtype=np.uint64)
    words = (stream.reshape(N, rw, 32) * weights[None, None, :]).sum(axis=2)
    return words.astype(np.uint32)


def unpack(packed: np.ndarray, K: int, d: int) -> np.ndarray:
    """Inverse of ``pack``: (N, row_words) uint32 -> (N, d/2) int64 (unclamped)."""
    packed = np.asarray(packed, dtype=np.uint32)
    N, rw = packed.shape
    B = index_bits(K)
    P = d // 2
    if B == 0:
        return np.zeros((N, P), dtype=np.int64)
    stream = (packed.astype(np.int64)[:, :, None] >> np.arange(32)[None, None, :]) & 1
    bits = stream.reshape(N, rw * 32)[:, : P * B].reshape(N, P, B)
    return (bits << np.arange(B)[None, None, :]).sum(axis=2)


# ---------------------------------------------------------------------------
# fp16 / bf16 rounding
# ---------------------------------------------------------------------------
def to_f16_bits(x: np.ndarray) -> np.ndarray:
    """fp64 -> IEEE binary16, round to nearest even, as uint16 bits."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def f16_bits_to_f64(u: np.ndarray) -> np.ndarray:
    return np.asarray(u, dtype=np.uint16).view(np.float16).astype(np.float64)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 (8 significant bits), round to nearest even, as uint16 bits.

    Normal range only (|x| in [2^-126, 2^127]) or zero; the codec's outputs stay
    inside it.  The rounding happens once, directly from fp64.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                       # x = m * 2^e, 0.5 <= |m| < 1
    q = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    return (q.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(u: np.ndarray) -> np.ndarray:
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# encode / decode
# ---------------------------------------------------------------------------
def encode(W: np.ndarray, s: np.ndarray, sigma: np.ndarray, b: int, sign_seed: int,
           C: np.ndarray, rows=None):
    """Encode rows of W given the calibration (s, sigma).

    Reading: the row norm is stored as fp16 (round to nearest even) metadata;
    the direction is normalised with the exact norm.
    Returns a dict with idx (M, d/2) int64, packed (M, row_words) uint32,
    rho (M,), rho_hat_bits (M,) uint16, zt (M, d/2, 2) and the fp64 distance
    diagnostics of ``nearest_centroid``.  ``rows`` selects a subset of rows.
    """
    W = np.asarray(W)
    if rows is not None:
        W = W[np.asarray(rows)]
    C = np.asarray(C, dtype=np.float32).reshape(-1, 2)
    K = C.shape[0]
    N, d = W.shape
    Zt, rho = normalized_pairs(W, s, sigma, b, sign_seed)
    idx = np.empty((N, d // 2), dtype=np.int64)
    d_at = np.empty((N, d // 2))
    d_best = np.empty((N, d // 2))
    d_second = np.empty((N, d // 2))
    for n in range(N):
        idx[n], d_at[n], d_best[n], d_second[n] = nearest_centroid(Zt[n], C)
    return {
        "idx": idx,
        "packed": pack(idx, K, d),
        "rho": rho,
        "rho_hat_bits": to_f16_bits(rho),
        "zt": Zt,
        "d64_at_idx": d_at,
        "d64_best": d_best,
        "d64_second": d_second,
    }


def inverse_scale(s) -> np.ndarray:
    """1 / s_j, taken as 0 where s_j = 0: a channel whose activations are all
    zero (r_j = 0, so s_j = 0 for alpha > 0) contributes nothing to a layer
    output, so its decoded weights and its activations are dropped."""
    s = np.asarray(s, dtype=np.float64)
    safe = np.where(s != 0.0, s, 1.0)
    return np.where(s != 0.0, 1.0 / safe, 0.0)


def decode(packed: np.ndarray, rho_hat_bits: np.ndarray, s, sigma: np.ndarray, b: int,
           sign_seed: int, C: np.ndarray, d: int) -> np.ndarray:
    """Decode (QAM-W, Methodology, Decoding): unpack, look up the centroids,
    multiply by sigma_k, undo the rotation, multiply by the stored row norm.

    Reading: decode also divides by s_j, returning an approximation of W; with
    s = None it stops at W' = W diag(s).  A column with s_j = 0 (an input
    channel whose activations are all zero, so that W' holds zeros there and
    its weights never reach the layer output) decodes as 0 rather than as a
    division by zero.  Indices >= K (impossible from ``encode``) are clamped
    to K - 1.  Returns fp64 (N, d).
    """
    C = np.asarray(C, dtype=np.float32).reshape(-1, 2).astype(np.float64)
    K = C.shape[0]
    idx = np.minimum(unpack(packed, K, d), K - 1)
    sigma = np.asarray(sigma, dtype=np.float64)
    N = idx.shape[0]
    Yh = np.empty((N, d))
    Yh[:, 0::2] = sigma[None, :] * C[idx, 0]
    Yh[:, 1::2] = sigma[None, :] * C[idx, 1]
    Uh = rotate_inverse(Yh, sign_mask(sign_seed, d), b)
    Wh = f16_bits_to_f64(rho_hat_bits)[:, None] * Uh
    if s is not None:
        Wh = Wh * inverse_scale(s)[None, :]
    return Wh


# ---------------------------------------------------------------------------
# decoded weights times activations
# ---------------------------------------------------------------------------
def decode_matmul(X: np.ndarray, packed: np.ndarray, rho_hat_bits: np.ndarray, s, sigma: np.ndarray,
                  b: int, sign_seed: int, C: np.ndarray, d: int) -> np.ndarray:
    """Y = X W^^T, W^ the decoded matrix: the layer output that the pages'
    pipeline computes after dequantising the weights (QAM-W, Methodology:
    Decoding; the dequantise-then-matmul inference path).  X is (T, d), the
    result (T, N), fp64: the plain definition, decode then multiply."""
    Wh = decode(packed, rho_hat_bits, s, sigma, b, sign_seed, C, d)
    return np.asarray(X, dtype=np.float64) @ Wh.T


def rotate_activations(X: np.ndarray, s, b: int, sign_seed: int) -> np.ndarray:
    """X~_t = R_fwd (X_t / s) for every activation row t (s = None means 1).

    Because a decoded row is W^_n = rho^_n (R_fwd^T y^_n) / s and R_fwd is
    orthogonal, <X_t, W^_n> = rho^_n <X~_t, y^_n>: a layer output can be
    formed from the rotated activations and the looked-up pairs
    y^_{n,2k:2k+2} = sigma_k C[idx_{n,k}] without undoing the rotation per
    weight row.  fp64 (T, d)."""
    X = np.asarray(X, dtype=np.float64)
    if s is not None:
        X = X * inverse_scale(s)[None, :]
    return rotate_forward(X, sign_mask(sign_seed, X.shape[1]), b)


def lookup_pairs(packed: np.ndarray, sigma: np.ndarray, C: np.ndarray, d: int) -> np.ndarray:
    """y^_n: the looked-up pairs sigma_k C[idx_{n,k}], interleaved, fp64 (N, d)."""
    C = np.asarray(C, dtype=np.float32).reshape(-1, 2).astype(np.float64)
    K = C.shape[0]
    idx = np.minimum(unpack(packed, K, d), K - 1)
    sigma = np.asarray(sigma, dtype=np.float64)
    Yh = np.empty((idx.shape[0], d))
    Yh[:, 0::2] = sigma[None, :] * C[idx, 0]
    Yh[:, 1::2] = sigma[None, :] * C[idx, 1]
    return Yh


# ---------------------------------------------------------------------------
# layer-output error
# ---------------------------------------------------------------------------
def output_error_direct(X: np.ndarray, dW: np.ndarray) -> float:
    """||X dW^T||_F^2 for activations X (n, d) and a weight error dW (m, d)."""
    E = np.asarray(X, dtype=np.float64) @ np.asarray(dW, dtype=np.float64).T
    return float(np.sum(E * E))


def output_error_trace(X: np.ndarray, dW: np.ndarray) -> float:
    """Tr(dW M dW^T) with M = X^T X, the second-moment form of the layer-output
    error (QAM-W, Methodology: the trace identity motivating the scaling).

    Reading: M is the unnormalised X^T X, the only form for which the identity
    holds as printed.
    """
    X = np.asarray(X, dtype=np.float64)
    dW = np.asarray(dW, dtype=np.float64)
    M = X.T @ X
    return float(np.trace(dW @ M @ dW.T))


def output_weighted_error(r: np.ndarray, dW: np.ndarray) -> float:
    """sum_j r_j^2 ||dW[:, j]||^2: the diagonal part of Tr(dW M dW^T) with
    M_jj = n r_j^2 (r_j the channel RMS), per activation row."""
    r = np.asarray(r, dtype=np.float64)
    dW = np.asarray(dW, dtype=np.float64)
    return float(np.sum((r * r)[None, :] * dW * dW))
