"""Seeded synthetic inputs for the QAM-W codec.

This module is the only code shared by the oracle's tests and the HIP path's
tests and benchmark.  It produces *inputs* only -- weight matrices, channel
RMS vectors and the Gaussian samples a codebook is trained on -- and holds
none of the codec's arithmetic (no scaling, rotation, quantisation or
packing).

The QAM-W pages evaluate on trained LLM checkpoints (TinyLlama-1.1B,
Qwen2.5-3B, Mistral-7B, Llama-2-7B and an unnamed 13B model).  None of those
weights exist here, so every workload below is a synthetic matrix with the
shape of an LLM linear layer of that size class and a stated distribution:
Gaussian or Student-t entries, optional outlier columns, and log-normal
channel RMS values.

Every generator is NumPy ``default_rng(seed)`` (PCG64).  bf16 matrices are
produced in fp32 and rounded to bf16 with round-to-nearest-even; they are
carried as ``uint16`` bit patterns because NumPy has no bf16 type.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import numpy as np

__all__ = [
    "Workload",
    "bf16_bits_from_f32",
    "bf16_bits_to_f32",
    "gaussian_samples",
    "matrix",
    "channel_rms",
    "activations",
    "get",
    "names",
    "stack_7b",
    "sha256",
]


# --------------------------------------------------------------------------
# bf16 helpers (input preparation only)
# --------------------------------------------------------------------------
def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even) -> uint16 bits.

    NaN inputs map to a quiet NaN; the generators never produce them.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        rounded = rounded.copy()
        rounded[nan] = np.uint16(0x7FC0)
    return rounded


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to fp32."""
    u = np.ascontiguousarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


# --------------------------------------------------------------------------
# primitive generators
# --------------------------------------------------------------------------
def gaussian_samples(n: int = 1 << 16, seed: int = 1) -> np.ndarray:
    """n draws of the unit circular Gaussian N(0, I_2), fp64, shape (n, 2).

    These are the training samples of the 2D codebook (the pages train it on
    the unit circular Gaussian, not on checkpoint data).
    """
    return np.random.default_rng(seed).standard_normal((n, 2))


def matrix(rows: int, cols: int, *, dist: str, std: float, seed: int,
           outlier_frac: float = 0.0, outlier_scale: float = 8.0,
           outlier_seed: Optional[int] = None) -> np.ndarray:
    """fp32 matrix (rows, cols) with entries of standard deviation ``std``.

    dist = "normal": N(0, std^2).
    dist = "t5":     Student-t with 5 degrees of freedom, scaled by
                     std / sqrt(5/3) so the entries have standard deviation std.
    outlier_frac:    round(outlier_frac * cols) columns, drawn without
                     replacement with ``outlier_seed``, are multiplied by
                     ``outlier_scale`` (in fp32, before any bf16 rounding).
    """
    rng = np.random.default_rng(seed)
    if dist == "normal":
        w = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(std)
    elif dist == "t5":
        w = (rng.standard_t(5.0, size=(rows, cols)) * (std / np.sqrt(5.0 / 3.0))).astype(np.float32)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    n_out = int(round(outlier_frac * cols))
    if n_out:
        cols_sel = np.random.default_rng(outlier_seed).choice(cols, size=n_out, replace=False)
        w[:, cols_sel] *= np.float32(outlier_scale)
    return w


def channel_rms(d: int, *, sigma_log: float, seed: int) -> np.ndarray:
    """Per-input-channel activation RMS r_j ~ LogNormal(0, sigma_log), fp32, all > 0."""
    return np.random.default_rng(seed).lognormal(0.0, sigma_log, size=d).astype(np.float32)


def activations(T: int, r: np.ndarray, *, seed: int) -> np.ndarray:
    """Synthetic layer inputs X (T, d) fp32: X[t, j] = r_j * g[t, j], g ~ N(0, 1).

    Channel j's activations have RMS r_j in expectation (the pages calibrate
    on real activations; these stand in for them with log-normal channel
    scales, the heavy-channel structure activation-aware scaling targets).
    """
    g = np.random.default_rng(seed).standard_normal((T, np.asarray(r).size))
    return (g * np.asarray(r, dtype=np.float64)[None, :]).astype(np.float32)


# --------------------------------------------------------------------------
# named workloads
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Workload:
    name: str
    W: np.ndarray            # fp32 values, or uint16 bf16 bit patterns when wdtype == "bf16"
    wdtype: str              # "f32" or "bf16"
    r: np.ndarray            # (d,) fp32 channel RMS
    alpha: float
    block: int
    sign_seed: int
    K: int

    @property
    def N(self) -> int:
        return int(self.W.shape[0])

    @property
    def d(self) -> int:
        return int(self.W.shape[1])

    def W_f32(self) -> np.ndarray:
        """The weight values as fp32 (exact for both storage types)."""
        return bf16_bits_to_f32(self.W) if self.wdtype == "bf16" else self.W


def _c1() -> Workload:
    W = matrix(256, 512, dist="normal", std=0.02, seed=100)
    r = channel_rms(512, sigma_log=0.5, seed=101)
    return Workload("c1_256x512", W, "f32", r, 0.5, 128, 0, 256)


def _c2() -> Workload:
    W = matrix(4096, 4096, dist="normal", std=0.02, seed=200,
               outlier_frac=0.01, outlier_scale=8.0, outlier_seed=202)
    r = channel_rms(4096, sigma_log=1.0, seed=201)
    return Workload("c2_4096x4096", bf16_bits_from_f32(W), "bf16", r, 0.5, 128, 0, 2048)


_C3_CACHE: dict = {}


def _c3_base() -> np.ndarray:
    if "W" not in _C3_CACHE:
        _C3_CACHE["W"] = bf16_bits_from_f32(
            matrix(11008, 4096, dist="t5", std=0.02, seed=300))
    return _C3_CACHE["W"]


def _c3() -> Workload:
    r = channel_rms(4096, sigma_log=1.2, seed=301)
    return Workload("c3_11008x4096", _c3_base(), "bf16", r, 0.5, 256, 0, 2048)


def _c3t() -> Workload:
    """The 4096 x 11008 down-projection shape: the exact transpose of c3's matrix."""
    W = np.ascontiguousarray(_c3_base().T)
    r = channel_rms(11008, sigma_log=1.2, seed=302)
    return Workload("c3t_4096x11008", W, "bf16", r, 0.5, 256, 0, 2048)


def _c4(K: int, alpha: float) -> Workload:
    W = matrix(5120, 13824, dist="normal", std=0.015, seed=400)
    r = channel_rms(13824, sigma_log=1.0, seed=401)
    return Workload(f"c4_5120x13824_K{K}_a{alpha:g}", bf16_bits_from_f32(W), "bf16",
                    r, alpha, 128, 0, K)


_STACK_SHAPES = {
    "q": (4096, 4096), "k": (4096, 4096), "v": (4096, 4096), "o": (4096, 4096),
    "gate": (11008, 4096), "up": (11008, 4096), "down": (4096, 11008),
}
_STACK_ORDER = ("q", "k", "v", "o", "gate", "up", "down")


def stack_7b(layer: int, proj: str) -> Workload:
    """One matrix of the 7B-shaped linear stack (32 layers x 7 projections)."""
    p = _STACK_ORDER.index(proj)
    rows, cols = _STACK_SHAPES[proj]
    W = matrix(rows, cols, dist="t5", std=0.02, seed=5000 + 8 * layer + p)
    r = channel_rms(cols, sigma_log=1.0, seed=6000 + 8 * layer + p)
    return Workload(f"c5_l{layer}_{proj}", bf16_bits_from_f32(W), "bf16", r, 0.5, 128, 0, 2048)


def names() -> list:
    out = ["c1_256x512", "c2_4096x4096", "c3_11008x4096", "c3t_4096x11008"]
    for K in (256, 1024, 2048, 4096):
        for a in (0.0, 0.5):
            out.append(f"c4_5120x13824_K{K}_a{a:g}")
    return out


def get(name: str) -> Workload:
    if name == "c1_256x512":
        return _c1()
    if name == "c2_4096x4096":
        return _c2()
    if name == "c3_11008x4096":
        return _c3()
    if name == "c3t_4096x11008":
        return _c3t()
    if name.startswith("c4_5120x13824_K"):
        k_part, a_part = name[len("c4_5120x13824_K"):].split("_a")
        return _c4(int(k_part), float(a_part))
    if name.startswith("c5_l"):
        layer, proj = name[len("c5_l"):].split("_", 1)
        return stack_7b(int(layer), proj)
    raise KeyError(name)
