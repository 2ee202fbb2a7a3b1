"""Python binding of the QAM-W C ABI over torch device tensors.

Each function has the name of the C entry point it calls and only marshals
arguments: it checks devices, dtypes and shapes, allocates the outputs and
workspace with torch when the caller passes none, and hands raw pointers plus
the current HIP stream to libqamw.so.  Every step of the codec runs in the
library's kernels.
"""
from __future__ import annotations

import json
import os
from typing import Optional

import numpy as np
import torch

from . import _lib

CODEBOOK_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "codebooks")

_WDT = {torch.float32: _lib.QAMW_F32, torch.bfloat16: _lib.QAMW_BF16}
_ODT = {torch.float32: _lib.QAMW_F32, torch.bfloat16: _lib.QAMW_BF16, torch.float16: _lib.QAMW_F16}


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t: torch.Tensor, name: str) -> None:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")


def _vec(t: torch.Tensor, name: str, n: int, dtype=torch.float32) -> None:
    _dev(t, name)
    if t.dtype != dtype or t.numel() != n or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor with {n} elements")


def _rows(W: torch.Tensor, name: str):
    _dev(W, name)
    if W.dim() != 2 or (W.stride(1) != 1 and W.shape[1] > 1):
        raise ValueError(f"{name} must be 2-D with unit column stride")
    # a single row's leading stride is arbitrary (torch and NumPy leave it so):
    # the row length is then its row pitch
    return W.shape[0], W.shape[1], (W.stride(0) if W.shape[0] > 1 else W.shape[1])


# ---------------------------------------------------------------- host helpers
def qamw_index_bits(K: int) -> int:
    return int(_lib.load().qamw_index_bits(K))


def qamw_packed_row_words(d: int, K: int) -> int:
    return int(_lib.load().qamw_packed_row_words(d, K))


def qamw_calibrate_workspace_bytes(N: int, d: int, block: int) -> int:
    return int(_lib.load().qamw_calibrate_workspace_bytes(N, d, block))


def qamw_encode_workspace_bytes(N: int, d: int) -> int:
    return int(_lib.load().qamw_encode_workspace_bytes(N, d))


def qamw_plan_bytes(K: int) -> int:
    return int(_lib.load().qamw_plan_bytes(K))


def _codebook(codebook: torch.Tensor) -> int:
    _dev(codebook, "codebook")
    if codebook.dtype != torch.float32 or codebook.dim() != 2 or codebook.shape[1] != 2 or not codebook.is_contiguous():
        raise ValueError("codebook must be a contiguous K x 2 float32 tensor")
    return codebook.shape[0]


def _workspace(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator returns 256-byte aligned blocks
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def load_codebook(K: int) -> np.ndarray:
    """The stored K x 2 float32 codebook (2D Lloyd-Max, unit circular Gaussian)."""
    path = os.path.join(CODEBOOK_DIR, f"qamw_K{K}.f32")
    with open(path, "rb") as f:
        C = np.frombuffer(f.read(), dtype="<f4").reshape(K, 2).copy()
    with open(os.path.join(CODEBOOK_DIR, f"qamw_K{K}.json")) as f:
        meta = json.load(f)
    if meta["K"] != K:
        raise ValueError(f"codebook metadata mismatch for K={K}")
    return C


def load_polar(Ka: int, Kp: int):
    """The stored polar code Ka x Kp: (levels [Ka], dirs [Kp][2], table [Ka Kp][2]), float32.

    ``table`` is the decode codebook: entry ia * Kp + ip = levels[ia] * dirs[ip]."""
    base = os.path.join(CODEBOOK_DIR, f"polar_A{Ka}_P{Kp}")
    with open(base + ".json") as f:
        meta = json.load(f)
    if (meta["Ka"], meta["Kp"]) != (Ka, Kp):
        raise ValueError(f"polar metadata mismatch for {Ka} x {Kp}")

    def read(name, shape):
        with open(name, "rb") as f:
            return np.frombuffer(f.read(), dtype="<f4").reshape(shape).copy()

    return read(base + "_levels.f32", (Ka,)), read(base + "_dirs.f32", (Kp, 2)), read(base + ".f32", (Ka * Kp, 2))


# ---------------------------------------------------------------- entry points
def qamw_build_plan(codebook: torch.Tensor, plan: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Nearest-centroid search plan for `codebook` (uint8 device buffer) for qamw_encode(plan=...)."""
    K = _codebook(codebook)
    need = qamw_plan_bytes(K)
    if need <= 0:
        raise ValueError(f"unsupported K={K}")
    if plan is None:
        plan = torch.empty(need, dtype=torch.uint8, device=codebook.device)
    _dev(plan, "plan")
    if plan.dtype != torch.uint8 or not plan.is_contiguous():
        raise ValueError("plan must be a contiguous uint8 tensor")
    _lib.check("qamw_build_plan", _lib.load().qamw_build_plan(
        codebook.data_ptr(), K, plan.data_ptr(), plan.numel(), _stream(stream)))
    return plan


def qamw_calibrate(W: torch.Tensor, chan_rms: torch.Tensor, alpha: float, block: int, sign_seed: int,
                   s_out: Optional[torch.Tensor] = None, sigma_out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None, stream=None):
    """Returns (s [d] fp32, sigma [d/2] fp32)."""
    N, d, ldw = _rows(W, "W")
    if W.dtype not in _WDT:
        raise ValueError("W must be float32 or bfloat16")
    _vec(chan_rms, "chan_rms", d)
    if s_out is None:
        s_out = torch.empty(d, dtype=torch.float32, device=W.device)
    if sigma_out is None:
        sigma_out = torch.empty(d // 2, dtype=torch.float32, device=W.device)
    _vec(s_out, "s_out", d)
    _vec(sigma_out, "sigma_out", d // 2)
    need = qamw_calibrate_workspace_bytes(N, d, block)
    if workspace is None:
        workspace = _workspace(need, W.device)
    _lib.check("qamw_calibrate", _lib.load().qamw_calibrate(
        W.data_ptr(), _WDT[W.dtype], N, d, ldw, chan_rms.data_ptr(), float(alpha), int(block),
        int(sign_seed), s_out.data_ptr(), sigma_out.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return s_out, sigma_out


def qamw_encode(W: torch.Tensor, s: torch.Tensor, sigma: torch.Tensor, block: int, sign_seed: int,
                codebook: torch.Tensor, plan: Optional[torch.Tensor] = None,
                packed: Optional[torch.Tensor] = None, rownorm_f16: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, stream=None):
    """Returns (packed [N][row_words] int32 holding uint32 words, rownorm [N] int16 holding fp16 bits).

    `plan` (from qamw_build_plan for the same codebook) speeds up the nearest-centroid
    search without changing the result; None searches the whole codebook."""
    N, d, ldw = _rows(W, "W")
    if W.dtype not in _WDT:
        raise ValueError("W must be float32 or bfloat16")
    _vec(s, "s", d)
    _vec(sigma, "sigma", d // 2)
    K = _codebook(codebook)
    rw = qamw_packed_row_words(d, K)
    if rw < 0:
        raise ValueError(f"unsupported K={K} or d={d}")
    if plan is not None:
        _dev(plan, "plan")
        if plan.dtype != torch.uint8 or plan.numel() < qamw_plan_bytes(K):
            raise ValueError("plan must be a uint8 tensor from qamw_build_plan for this K")
    if packed is None:
        packed = torch.empty((N, rw), dtype=torch.int32, device=W.device)
    if rownorm_f16 is None:
        rownorm_f16 = torch.empty(N, dtype=torch.int16, device=W.device)
    _dev(packed, "packed")
    if packed.dtype != torch.int32 or tuple(packed.shape) != (N, rw) or not packed.is_contiguous():
        raise ValueError(f"packed must be a contiguous int32 tensor of shape ({N}, {rw})")
    _vec(rownorm_f16, "rownorm_f16", N, torch.int16)
    need = qamw_encode_workspace_bytes(N, d)
    if workspace is None:
        workspace = _workspace(need, W.device)
    _lib.check("qamw_encode", _lib.load().qamw_encode(
        W.data_ptr(), _WDT[W.dtype], N, d, ldw, s.data_ptr(), sigma.data_ptr(), int(block), int(sign_seed),
        codebook.data_ptr(), K, None if plan is None else plan.data_ptr(), 0 if plan is None else plan.numel(),
        packed.data_ptr(), rownorm_f16.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return packed, rownorm_f16


def qamw_encode_noalloc(W: torch.Tensor, s: torch.Tensor, sigma: torch.Tensor, block: int, sign_seed: int,
                        codebook: torch.Tensor, plan: Optional[torch.Tensor] = None,
                        packed: Optional[torch.Tensor] = None, rownorm_f16: Optional[torch.Tensor] = None,
                        stream=None):
    """qamw_encode with the library's own per-GPU workspace (no workspace argument; the C call
    allocates nothing).  Returns (packed, rownorm_f16); pass both to avoid allocating them here."""
    N, d, ldw = _rows(W, "W")
    if W.dtype not in _WDT:
        raise ValueError("W must be float32 or bfloat16")
    _vec(s, "s", d)
    _vec(sigma, "sigma", d // 2)
    K = _codebook(codebook)
    rw = qamw_packed_row_words(d, K)
    if rw < 0:
        raise ValueError(f"unsupported K={K} or d={d}")
    if plan is not None:
        _dev(plan, "plan")
        if plan.dtype != torch.uint8 or plan.numel() < qamw_plan_bytes(K):
            raise ValueError("plan must be a uint8 tensor from qamw_build_plan for this K")
    if packed is None:
        packed = torch.empty((N, rw), dtype=torch.int32, device=W.device)
    if rownorm_f16 is None:
        rownorm_f16 = torch.empty(N, dtype=torch.int16, device=W.device)
    _dev(packed, "packed")
    if packed.dtype != torch.int32 or tuple(packed.shape) != (N, rw) or not packed.is_contiguous():
        raise ValueError(f"packed must be a contiguous int32 tensor of shape ({N}, {rw})")
    _vec(rownorm_f16, "rownorm_f16", N, torch.int16)
    _lib.check("qamw_encode_noalloc", _lib.load().qamw_encode_noalloc(
        W.data_ptr(), _WDT[W.dtype], N, d, ldw, s.data_ptr(), sigma.data_ptr(), int(block), int(sign_seed),
        codebook.data_ptr(), K, None if plan is None else plan.data_ptr(), 0 if plan is None else plan.numel(),
        packed.data_ptr(), rownorm_f16.data_ptr(), _stream(stream)))
    return packed, rownorm_f16


def qamw_calibrate_encode_workspace_bytes(N: int, d: int) -> int:
    return int(_lib.load().qamw_calibrate_encode_workspace_bytes(N, d))


def qamw_calibrate_prepare(W: torch.Tensor, chan_rms: torch.Tensor, alpha: float, block: int, sign_seed: int,
                           s_out: Optional[torch.Tensor] = None, sigma_out: Optional[torch.Tensor] = None,
                           rownorm_f16: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                           stream=None):
    """The calibration half of qamw_calibrate_encode: returns (s, sigma, rownorm_f16, workspace), the
    workspace ready for qamw_encode_indices (same packed words as qamw_calibrate_encode)."""
    N, d, ldw = _rows(W, "W")
    if W.dtype not in _WDT:
        raise ValueError("W must be float32 or bfloat16")
    _vec(chan_rms, "chan_rms", d)
    if s_out is None:
        s_out = torch.empty(d, dtype=torch.float32, device=W.device)
    if sigma_out is None:
        sigma_out = torch.empty(d // 2, dtype=torch.float32, device=W.device)
    if rownorm_f16 is None:
        rownorm_f16 = torch.empty(N, dtype=torch.int16, device=W.device)
    _vec(s_out, "s_out", d)
    _vec(sigma_out, "sigma_out", d // 2)
    _vec(rownorm_f16, "rownorm_f16", N, torch.int16)
    if workspace is None:
        workspace = _workspace(qamw_calibrate_encode_workspace_bytes(N, d), W.device)
    _dev(workspace, "workspace")
    _lib.check("qamw_calibrate_prepare", _lib.load().qamw_calibrate_prepare(
        W.data_ptr(), _WDT[W.dtype], N, d, ldw, chan_rms.data_ptr(), float(alpha), int(block), int(sign_seed),
        s_out.data_ptr(), sigma_out.data_ptr(), rownorm_f16.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return s_out, sigma_out, rownorm_f16, workspace


def qamw_calibrate_encode(W: torch.Tensor, chan_rms: torch.Tensor, alpha: float, block: int, sign_seed: int,
                          codebook: torch.Tensor, plan: Optional[torch.Tensor] = None,
                          s_out: Optional[torch.Tensor] = None, sigma_out: Optional[torch.Tensor] = None,
                          packed: Optional[torch.Tensor] = None, rownorm_f16: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None, stream=None):
    """qamw_calibrate + qamw_encode in one call sharing the row norms:
    returns (s, sigma, packed, rownorm_f16), bit-identical to the two calls."""
    N, d, ldw = _rows(W, "W")
    if W.dtype not in _WDT:
        raise ValueError("W must be float32 or bfloat16")
    _vec(chan_rms, "chan_rms", d)
    K = _codebook(codebook)
    rw = qamw_packed_row_words(d, K)
    if rw < 0:
        raise ValueError(f"unsupported K={K} or d={d}")
    if plan is not None:
        _dev(plan, "plan")
        if plan.dtype != torch.uint8 or plan.numel() < qamw_plan_bytes(K):
            raise ValueError("plan must be a uint8 tensor from qamw_build_plan for this K")
    if s_out is None:
        s_out = torch.empty(d, dtype=torch.float32, device=W.device)
    if sigma_out is None:
        sigma_out = torch.empty(d // 2, dtype=torch.float32, device=W.device)
    if packed is None:
        packed = torch.empty((N, rw), dtype=torch.int32, device=W.device)
    if rownorm_f16 is None:
        rownorm_f16 = torch.empty(N, dtype=torch.int16, device=W.device)
    _vec(s_out, "s_out", d)
    _vec(sigma_out, "sigma_out", d // 2)
    _dev(packed, "packed")
    if packed.dtype != torch.int32 or tuple(packed.shape) != (N, rw) or not packed.is_contiguous():
        raise ValueError(f"packed must be a contiguous int32 tensor of shape ({N}, {rw})")
    _vec(rownorm_f16, "rownorm_f16", N, torch.int16)
    if workspace is None:
        workspace = _workspace(qamw_calibrate_encode_workspace_bytes(N, d), W.device)
    _lib.check("qamw_calibrate_encode", _lib.load().qamw_calibrate_encode(
        W.data_ptr(), _WDT[W.dtype], N, d, ldw, chan_rms.data_ptr(), float(alpha), int(block), int(sign_seed),
        codebook.data_ptr(), K, None if plan is None else plan.data_ptr(), 0 if plan is None else plan.numel(),
        s_out.data_ptr(), sigma_out.data_ptr(),
        packed.data_ptr(), rownorm_f16.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return s_out, sigma_out, packed, rownorm_f16


def qamw_encode_prepare(W: torch.Tensor, s: torch.Tensor, sigma: torch.Tensor, block: int, sign_seed: int,
                        rownorm_f16: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                        stream=None):
    """Encode phase 1: returns (rownorm [N] int16 holding fp16 bits, workspace for qamw_encode_indices)."""
    N, d, ldw = _rows(W, "W")
    if W.dtype not in _WDT:
        raise ValueError("W must be float32 or bfloat16")
    _vec(s, "s", d)
    _vec(sigma, "sigma", d // 2)
    if rownorm_f16 is None:
        rownorm_f16 = torch.empty(N, dtype=torch.int16, device=W.device)
    _vec(rownorm_f16, "rownorm_f16", N, torch.int16)
    if workspace is None:
        workspace = _workspace(qamw_encode_workspace_bytes(N, d), W.device)
    _lib.check("qamw_encode_prepare", _lib.load().qamw_encode_prepare(
        W.data_ptr(), _WDT[W.dtype], N, d, ldw, s.data_ptr(), sigma.data_ptr(), int(block), int(sign_seed),
        rownorm_f16.data_ptr(), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return rownorm_f16, workspace


def qamw_encode_indices(W: torch.Tensor, block: int, codebook: torch.Tensor, workspace: torch.Tensor,
                        plan: Optional[torch.Tensor] = None, packed: Optional[torch.Tensor] = None, stream=None):
    """Encode phase 2 from a workspace filled by qamw_encode_prepare: returns packed [N][row_words] int32."""
    N, d, ldw = _rows(W, "W")
    if W.dtype not in _WDT:
        raise ValueError("W must be float32 or bfloat16")
    K = _codebook(codebook)
    rw = qamw_packed_row_words(d, K)
    if rw < 0:
        raise ValueError(f"unsupported K={K} or d={d}")
    if plan is not None:
        _dev(plan, "plan")
        if plan.dtype != torch.uint8 or plan.numel() < qamw_plan_bytes(K):
            raise ValueError("plan must be a uint8 tensor from qamw_build_plan for this K")
    if packed is None:
        packed = torch.empty((N, rw), dtype=torch.int32, device=W.device)
    _dev(packed, "packed")
    if packed.dtype != torch.int32 or tuple(packed.shape) != (N, rw) or not packed.is_contiguous():
        raise ValueError(f"packed must be a contiguous int32 tensor of shape ({N}, {rw})")
    _dev(workspace, "workspace")
    _lib.check("qamw_encode_indices", _lib.load().qamw_encode_indices(
        W.data_ptr(), _WDT[W.dtype], N, d, ldw, int(block), codebook.data_ptr(), K,
        None if plan is None else plan.data_ptr(), 0 if plan is None else plan.numel(), packed.data_ptr(),
        workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return packed


def qamw_lloyd_workspace_bytes(K: int) -> int:
    return int(_lib.load().qamw_lloyd_workspace_bytes(K))


def qamw_lloyd_update(W: torch.Tensor, block: int, packed: torch.Tensor, codebook: torch.Tensor,
                      enc_workspace: torch.Tensor, out: Optional[torch.Tensor] = None,
                      distortion: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                      stream=None):
    """One Lloyd update on the matrix's normalised pairs: returns (codebook' [K][2] fp32,
    distortion [1] fp64 of the assignment in packed)."""
    N, d, ldw = _rows(W, "W")
    if W.dtype not in _WDT:
        raise ValueError("W must be float32 or bfloat16")
    K = _codebook(codebook)
    rw = qamw_packed_row_words(d, K)
    _dev(packed, "packed")
    if packed.dtype != torch.int32 or tuple(packed.shape) != (N, rw) or not packed.is_contiguous():
        raise ValueError(f"packed must be a contiguous int32 tensor of shape ({N}, {rw})")
    _dev(enc_workspace, "enc_workspace")
    if out is None:
        out = torch.empty((K, 2), dtype=torch.float32, device=W.device)
    if distortion is None:
        distortion = torch.empty(1, dtype=torch.float64, device=W.device)
    if workspace is None:
        workspace = _workspace(qamw_lloyd_workspace_bytes(K), W.device)
    _lib.check("qamw_lloyd_update", _lib.load().qamw_lloyd_update(
        W.data_ptr(), _WDT[W.dtype], N, d, ldw, int(block), packed.data_ptr(), codebook.data_ptr(), K,
        enc_workspace.data_ptr(), enc_workspace.numel() * enc_workspace.element_size(), out.data_ptr(),
        distortion.data_ptr(), workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, distortion


def qamw_learn_codebook(W: torch.Tensor, block: int, enc_workspace: torch.Tensor, codebook_init: torch.Tensor,
                        iters: int, out: Optional[torch.Tensor] = None, distortion: Optional[torch.Tensor] = None,
                        plan: Optional[torch.Tensor] = None, packed: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None, stream=None):
    """iters Lloyd rounds on the matrix's own pairs from codebook_init: returns (codebook [K][2] fp32,
    distortion [iters] fp64, round t's mean squared distance)."""
    N, d, ldw = _rows(W, "W")
    if W.dtype not in _WDT:
        raise ValueError("W must be float32 or bfloat16")
    K = _codebook(codebook_init)
    rw = qamw_packed_row_words(d, K)
    _dev(enc_workspace, "enc_workspace")
    if out is None:
        out = torch.empty((K, 2), dtype=torch.float32, device=W.device)
    if distortion is None:
        distortion = torch.empty(int(iters), dtype=torch.float64, device=W.device)
    if plan is None:
        plan = torch.empty(qamw_plan_bytes(K), dtype=torch.uint8, device=W.device)
    if packed is None:
        packed = torch.empty((N, rw), dtype=torch.int32, device=W.device)
    if workspace is None:
        workspace = _workspace(qamw_lloyd_workspace_bytes(K), W.device)
    _lib.check("qamw_learn_codebook", _lib.load().qamw_learn_codebook(
        W.data_ptr(), _WDT[W.dtype], N, d, ldw, int(block), enc_workspace.data_ptr(),
        enc_workspace.numel() * enc_workspace.element_size(), codebook_init.data_ptr(), K, int(iters),
        out.data_ptr(), distortion.data_ptr(), plan.data_ptr(), plan.numel(), packed.data_ptr(),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, distortion


def qamw_encode_polar(W: torch.Tensor, s: torch.Tensor, sigma: torch.Tensor, block: int, sign_seed: int,
                      levels: torch.Tensor, dirs: torch.Tensor, packed: Optional[torch.Tensor] = None,
                      rownorm_f16: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                      stream=None):
    """Polar-code encode: returns (packed [N][row_words] int32, rownorm [N] int16 holding fp16 bits);
    indices ia * Kp + ip decode with the Ka Kp-entry table of ``load_polar``."""
    N, d, ldw = _rows(W, "W")
    if W.dtype not in _WDT:
        raise ValueError("W must be float32 or bfloat16")
    _vec(s, "s", d)
    _vec(sigma, "sigma", d // 2)
    _dev(levels, "levels")
    if levels.dtype != torch.float32 or levels.dim() != 1 or not levels.is_contiguous():
        raise ValueError("levels must be a contiguous 1-D float32 tensor")
    Ka = levels.shape[0]
    Kp = _codebook(dirs)
    rw = qamw_packed_row_words(d, Ka * Kp)
    if rw < 0:
        raise ValueError(f"unsupported Ka x Kp = {Ka} x {Kp} or d={d}")
    if packed is None:
        packed = torch.empty((N, rw), dtype=torch.int32, device=W.device)
    if rownorm_f16 is None:
        rownorm_f16 = torch.empty(N, dtype=torch.int16, device=W.device)
    _dev(packed, "packed")
    if packed.dtype != torch.int32 or tuple(packed.shape) != (N, rw) or not packed.is_contiguous():
        raise ValueError(f"packed must be a contiguous int32 tensor of shape ({N}, {rw})")
    _vec(rownorm_f16, "rownorm_f16", N, torch.int16)
    if workspace is None:
        workspace = _workspace(qamw_encode_workspace_bytes(N, d), W.device)
    _lib.check("qamw_encode_polar", _lib.load().qamw_encode_polar(
        W.data_ptr(), _WDT[W.dtype], N, d, ldw, s.data_ptr(), sigma.data_ptr(), int(block), int(sign_seed),
        levels.data_ptr(), Ka, dirs.data_ptr(), Kp, packed.data_ptr(), rownorm_f16.data_ptr(),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(stream)))
    return packed, rownorm_f16


def qamw_channel_rms_workspace_bytes(T: int, d: int) -> int:
    return int(_lib.load().qamw_channel_rms_workspace_bytes(T, d))


def qamw_output_error_workspace_bytes(T: int, N: int, d: int) -> int:
    return int(_lib.load().qamw_output_error_workspace_bytes(T, N, d))


def qamw_channel_rms(X: torch.Tensor, out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """r_j = sqrt(mean_t X[t][j]^2) of T activation rows X [T][d]: the chan_rms input of qamw_calibrate."""
    T, d, ldx = _rows(X, "X")
    if X.dtype not in _WDT:
        raise ValueError("X must be float32 or bfloat16")
    if out is None:
        out = torch.empty(d, dtype=torch.float32, device=X.device)
    _vec(out, "out", d)
    if workspace is None:
        workspace = _workspace(qamw_channel_rms_workspace_bytes(T, d), X.device)
    _lib.check("qamw_channel_rms", _lib.load().qamw_channel_rms(
        X.data_ptr(), _WDT[X.dtype], T, d, ldx, out.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def qamw_output_error(X: torch.Tensor, W: torch.Tensor, W_hat: torch.Tensor, out: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """E = || X (W - W_hat)^T ||_F^2 = Tr(dW X^T X dW^T) as a one-element float64 device tensor."""
    T, d, ldx = _rows(X, "X")
    N, d2, ldw = _rows(W, "W")
    N2, d3, ldh = _rows(W_hat, "W_hat")
    if (d2, d3, N2) != (d, d, N):
        raise ValueError("X [T][d], W [N][d] and W_hat [N][d] must agree")
    for t, name in ((X, "X"), (W, "W"), (W_hat, "W_hat")):
        if t.dtype not in _WDT:
            raise ValueError(f"{name} must be float32 or bfloat16")
    if out is None:
        out = torch.empty(1, dtype=torch.float64, device=X.device)
    _vec(out, "out", 1, torch.float64)
    if workspace is None:
        workspace = _workspace(qamw_output_error_workspace_bytes(T, N, d), X.device)
    _lib.check("qamw_output_error", _lib.load().qamw_output_error(
        X.data_ptr(), _WDT[X.dtype], T, d, ldx, W.data_ptr(), _WDT[W.dtype], N, ldw, W_hat.data_ptr(),
        _WDT[W_hat.dtype], ldh, out.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def qamw_decode(packed: torch.Tensor, rownorm_f16: torch.Tensor, d: int, s: Optional[torch.Tensor],
                sigma: torch.Tensor, block: int, sign_seed: int, codebook: torch.Tensor,
                out_dtype=torch.float32, out: Optional[torch.Tensor] = None, stream=None):
    """Returns the decoded [N][d] matrix in out_dtype (fp32, bf16 or fp16)."""
    _dev(packed, "packed")
    N = packed.shape[0]
    K = _codebook(codebook)
    rw = qamw_packed_row_words(d, K)
    if packed.dtype != torch.int32 or tuple(packed.shape) != (N, rw) or not packed.is_contiguous():
        raise ValueError(f"packed must be a contiguous int32 tensor of shape ({N}, {rw})")
    _vec(rownorm_f16, "rownorm_f16", N, torch.int16)
    if s is not None:
        _vec(s, "s", d)
    _vec(sigma, "sigma", d // 2)
    if out is None:
        out = torch.empty((N, d), dtype=out_dtype, device=packed.device)
    n2, d2, ldo = _rows(out, "out")
    if (n2, d2) != (N, d) or out.dtype not in _ODT:
        raise ValueError("out must be N x d of float32, bfloat16 or float16")
    _lib.check("qamw_decode", _lib.load().qamw_decode(
        packed.data_ptr(), rownorm_f16.data_ptr(), N, d, None if s is None else s.data_ptr(),
        sigma.data_ptr(), int(block), int(sign_seed), codebook.data_ptr(), K, out.data_ptr(),
        _ODT[out.dtype], ldo, _stream(stream)))
    return out


def qamw_rotate_activations(X: torch.Tensor, s: Optional[torch.Tensor], block: int, sign_seed: int,
                            out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Xr = bf16(R_fwd (X / s)) per activation row: the left operand of qamw_decode_matmul."""
    T, d, ldx = _rows(X, "X")
    if X.dtype not in _WDT:
        raise ValueError("X must be float32 or bfloat16")
    if s is not None:
        _vec(s, "s", d)
    if out is None:
        out = torch.empty((T, d), dtype=torch.bfloat16, device=X.device)
    t2, d2, ldr = _rows(out, "out")
    if (t2, d2) != (T, d) or out.dtype != torch.bfloat16:
        raise ValueError("out must be a T x d bfloat16 tensor")
    _lib.check("qamw_rotate_activations", _lib.load().qamw_rotate_activations(
        X.data_ptr(), _WDT[X.dtype], T, d, ldx, None if s is None else s.data_ptr(), int(block), int(sign_seed),
        out.data_ptr(), ldr, _stream(stream)))
    return out


def qamw_decode_matmul(Xr: torch.Tensor, packed: torch.Tensor, rownorm_f16: torch.Tensor, sigma: torch.Tensor,
                       codebook: torch.Tensor, out_dtype=torch.float32, out: Optional[torch.Tensor] = None,
                       stream=None) -> torch.Tensor:
    """Y = X W^^T [T][N] from rotated activations (qamw_rotate_activations) and the packed matrix."""
    T, d, ldr = _rows(Xr, "Xr")
    if Xr.dtype != torch.bfloat16:
        raise ValueError("Xr must be bfloat16 (from qamw_rotate_activations)")
    _dev(packed, "packed")
    N = packed.shape[0]
    K = _codebook(codebook)
    rw = qamw_packed_row_words(d, K)
    if packed.dtype != torch.int32 or tuple(packed.shape) != (N, rw) or not packed.is_contiguous():
        raise ValueError(f"packed must be a contiguous int32 tensor of shape ({N}, {rw})")
    _vec(rownorm_f16, "rownorm_f16", N, torch.int16)
    _vec(sigma, "sigma", d // 2)
    if out is None:
        out = torch.empty((T, N), dtype=out_dtype, device=Xr.device)
    t2, n2, ldy = _rows(out, "out")
    if (t2, n2) != (T, N) or out.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out must be T x N of float32 or bfloat16")
    _lib.check("qamw_decode_matmul", _lib.load().qamw_decode_matmul(
        Xr.data_ptr(), T, d, ldr, packed.data_ptr(), rownorm_f16.data_ptr(), N, sigma.data_ptr(),
        codebook.data_ptr(), K, out.data_ptr(), _ODT[out.dtype], ldy, _stream(stream)))
    return out
