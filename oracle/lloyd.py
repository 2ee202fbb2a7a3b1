"""2D Lloyd-Max codebook trainer, fp64 (test infrastructure only).

The codec uses one 2D Lloyd-Max codebook trained on the unit circular
Gaussian, not on checkpoint data (QAM-W, Methodology, Joint 2D Quantization;
Significance and Claims, on the synthetic codebook).  Lloyd's algorithm
alternates two steps on a fixed training sample: assign each sample to its
nearest centroid, then move each centroid to the mean of its cell.

Readings (the pages give no training details):
  * samples: 2^16 draws of N(0, I_2), seed 1 (passed in by the caller);
  * initial centroids: the first K samples;
  * exactly ``iters`` (50) assign/update rounds; ties to the lowest index;
  * a centroid whose cell is empty stays where it is;
  * centroids are stored as fp32 after the last update.
"""
from __future__ import annotations

import numpy as np


def assign(X: np.ndarray, C: np.ndarray, chunk: int = 2048):
    """Nearest-centroid assignment of samples X (n, 2) to C (K, 2), fp64.

    Returns (idx (n,) int64, squared distance to the chosen centroid (n,)).
    """
    X = np.asarray(X, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    n = X.shape[0]
    idx = np.empty(n, dtype=np.int64)
    dmin = np.empty(n)
    for a in range(0, n, chunk):
        x = X[a:a + chunk]
        D = (x[:, 0:1] - C[None, :, 0]) ** 2 + (x[:, 1:2] - C[None, :, 1]) ** 2
        i = np.argmin(D, axis=1)
        idx[a:a + chunk] = i
        dmin[a:a + chunk] = D[np.arange(x.shape[0]), i]
    return idx, dmin


def cell_means(X: np.ndarray, idx: np.ndarray, K: int):
    """Per-cell sample mean and count.  Cells with no sample get mean NaN."""
    X = np.asarray(X, dtype=np.float64)
    cnt = np.bincount(idx, minlength=K).astype(np.float64)
    sx = np.bincount(idx, weights=X[:, 0], minlength=K)
    sy = np.bincount(idx, weights=X[:, 1], minlength=K)
    with np.errstate(invalid="ignore", divide="ignore"):
        mean = np.stack([sx / cnt, sy / cnt], axis=1)
    return mean, cnt


def train(X: np.ndarray, K: int, iters: int = 50):
    """Lloyd iterations from the first K samples.

    Returns (C fp64 (K, 2), history) where history[t] is the mean squared
    distortion of the assignment made in round t (t < iters) and
    history[iters] the distortion of the returned centroids.  Stored
    codebooks are these centroids rounded to fp32.
    """
    X = np.asarray(X, dtype=np.float64)
    if X.shape[0] < K:
        raise ValueError("need at least K samples")
    C = X[:K].copy()
    history = []
    for _ in range(iters):
        idx, dmin = assign(X, C)
        history.append(float(dmin.mean()))
        mean, cnt = cell_means(X, idx, K)
        C = np.where(cnt[:, None] > 0, mean, C)
    _, dmin = assign(X, C)
    history.append(float(dmin.mean()))
    return C, history


def refine_on_pairs(Zt: np.ndarray, C0: np.ndarray, iters: int):
    """Lloyd rounds on a matrix's own normalised pairs, from a given codebook.

    The pages train the codebook once on the unit circular Gaussian and
    suggest that a codebook learned from a checkpoint's own pair
    distribution could do better (QAM-W, Significance and Claims, on the
    synthetic codebook).  Reading: start from the stored Gaussian codebook
    and run Lloyd rounds on the pairs z~ the encoder quantises.  Each round
    assigns every pair with the codec's own nearest-centroid rule -- decided
    in fp32, lowest index on ties (``qamw_ref.nearest_centroid``) -- then
    moves each centroid to the fp64 mean of its pairs, rounded to fp32; an
    empty cell keeps its centroid.

    Zt: (M, 2) fp64 pairs; C0: (K, 2) fp32.  Returns (C fp32 (K, 2) after
    ``iters`` rounds, history) with history[t] the fp64 mean squared
    distance of round t's assignment to round t's codebook.
    """
    from oracle import qamw_ref as O

    Z = np.asarray(Zt, dtype=np.float64).reshape(-1, 2)
    C = np.asarray(C0, dtype=np.float32).reshape(-1, 2).copy()
    K = C.shape[0]
    history = []
    for _ in range(iters):
        idx = np.empty(Z.shape[0], dtype=np.int64)
        for a in range(0, Z.shape[0], 4096):
            idx[a:a + 4096] = O.nearest_centroid(Z[a:a + 4096], C)[0]
        C64 = C.astype(np.float64)
        history.append(float(np.mean(np.sum((Z - C64[idx]) ** 2, axis=1))))
        mean, cnt = cell_means(Z, idx, K)
        C = np.where(cnt[:, None] > 0, mean, C64).astype(np.float32)
    return C, history
