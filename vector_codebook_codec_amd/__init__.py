"""QAM-W weight codec on AMD Instinct MI355X (gfx950).

The codec's work runs in hand-written HIP kernels behind the C ABI of
include/qamw.h (libqamw.so, built in-tree by ``_build.build()``).  This
package binds that ABI for torch device tensors; see ``codec`` for the entry
points ``qamw_calibrate``, ``qamw_encode`` and ``qamw_decode``.
"""
from .codec import (  # noqa: F401
    load_codebook,
    load_polar,
    qamw_build_plan,
    qamw_calibrate,
    qamw_calibrate_encode,
    qamw_calibrate_prepare,
    qamw_calibrate_encode_workspace_bytes,
    qamw_calibrate_workspace_bytes,
    qamw_channel_rms,
    qamw_channel_rms_workspace_bytes,
    qamw_decode,
    qamw_decode_matmul,
    qamw_encode,
    qamw_encode_noalloc,
    qamw_encode_indices,
    qamw_encode_polar,
    qamw_encode_prepare,
    qamw_encode_workspace_bytes,
    qamw_index_bits,
    qamw_learn_codebook,
    qamw_lloyd_update,
    qamw_lloyd_workspace_bytes,
    qamw_output_error,
    qamw_output_error_workspace_bytes,
    qamw_packed_row_words,
    qamw_plan_bytes,
    qamw_rotate_activations,
)

__version__ = "0.1.0"
