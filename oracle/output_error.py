"""Calibration statistics of the activations and the layer-output error,
fp64 definitions (test infrastructure only).

QAM-W, Methodology: Activation-Aware Scaling -- r_j is the RMS of input
channel j's activations; and the composite bound chain's trace identity,
which ties the layer-output error to the weight error through the
activations' second-moment matrix:

    || X dW^T ||_F^2 = Tr(dW M dW^T),   M = X^T X,   dW = W - W^.

Reading: M is the unnormalised X^T X (the only reading under which the
printed identity holds as written), so r_j^2 = M_jj / T for T rows of X.
"""
from __future__ import annotations

import numpy as np


def channel_rms(X: np.ndarray) -> np.ndarray:
    """r_j = sqrt(mean_t X[t, j]^2), fp64 (d,)."""
    X = np.asarray(X, dtype=np.float64)
    return np.sqrt(np.mean(X * X, axis=0))


def gram(X: np.ndarray) -> np.ndarray:
    """M = X^T X, fp64 (d, d)."""
    X = np.asarray(X, dtype=np.float64)
    return X.T @ X


def output_error(W: np.ndarray, W_hat: np.ndarray, X: np.ndarray) -> float:
    """E_out = Tr(dW M dW^T) with dW = W - W_hat and M = X^T X, in fp64.

    Written as the trace of the product the identity names; dW M dW^T is
    formed row block by row block to bound memory.
    """
    dW = np.asarray(W, dtype=np.float64) - np.asarray(W_hat, dtype=np.float64)
    M = gram(X)
    tot = 0.0
    for a in range(0, dW.shape[0], 256):
        blk = dW[a:a + 256]
        tot += float(np.einsum("ij,ij->", blk @ M, blk))      # sum_i (dW_i M dW_i^T)
    return tot
