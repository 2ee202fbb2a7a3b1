"""ctypes binding of libqamw.so: the C ABI of include/qamw.h, name for name.

Loading fails loudly when the library has not been built; there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

from ._build import LIB_PATH

QAMW_OK, QAMW_EINVAL, QAMW_EUNSUPPORTED, QAMW_EHIP, QAMW_EWORKSPACE = 0, -1, -2, -3, -4
QAMW_F32, QAMW_BF16, QAMW_F16 = 0, 1, 2

_c = ctypes
_p = _c.c_void_p
_i32, _i64, _u64, _f32, _sz = _c.c_int32, _c.c_int64, _c.c_uint64, _c.c_float, _c.c_size_t

SIGNATURES = {
    "qamw_index_bits": (_i32, [_i32]),
    "qamw_packed_row_words": (_i64, [_i64, _i32]),
    "qamw_calibrate_workspace_bytes": (_sz, [_i64, _i64, _i32]),
    "qamw_encode_workspace_bytes": (_sz, [_i64, _i64]),
    "qamw_status_string": (_c.c_char_p, [_i32]),
    "qamw_last_error": (_c.c_char_p, []),
    "qamw_version": (_c.c_char_p, []),
    "qamw_calibrate": (_i32, [_p, _i32, _i64, _i64, _i64, _p, _f32, _i32, _u64, _p, _p, _p, _sz, _p]),
    "qamw_plan_bytes": (_sz, [_i32]),
    "qamw_build_plan": (_i32, [_p, _i32, _p, _sz, _p]),
    "qamw_encode": (_i32, [_p, _i32, _i64, _i64, _i64, _p, _p, _i32, _u64, _p, _i32, _p, _sz, _p, _p, _p, _sz,
                         _p]),
    "qamw_encode_noalloc_scratch_bytes": (_sz, []),
    "qamw_encode_noalloc": (_i32, [_p, _i32, _i64, _i64, _i64, _p, _p, _i32, _u64, _p, _i32, _p, _sz, _p, _p, _p]),
    "qamw_encode_prepare": (_i32, [_p, _i32, _i64, _i64, _i64, _p, _p, _i32, _u64, _p, _p, _sz, _p]),
    "qamw_encode_indices": (_i32, [_p, _i32, _i64, _i64, _i64, _i32, _p, _i32, _p, _sz, _p, _p, _sz, _p]),
    "qamw_calibrate_encode_workspace_bytes": (_sz, [_i64, _i64]),
    "qamw_calibrate_prepare": (_i32, [_p, _i32, _i64, _i64, _i64, _p, _f32, _i32, _u64, _p, _p, _p, _p, _sz, _p]),
    "qamw_calibrate_encode": (_i32, [_p, _i32, _i64, _i64, _i64, _p, _f32, _i32, _u64, _p, _i32, _p, _sz, _p, _p, _p,
                                     _p, _p, _sz, _p]),
    "qamw_lloyd_workspace_bytes": (_sz, [_i32]),
    "qamw_lloyd_update": (_i32, [_p, _i32, _i64, _i64, _i64, _i32, _p, _p, _i32, _p, _sz, _p, _p, _p, _sz, _p]),
    "qamw_learn_codebook": (_i32, [_p, _i32, _i64, _i64, _i64, _i32, _p, _sz, _p, _i32, _i32, _p, _p, _p, _sz, _p,
                                   _p, _sz, _p]),
    "qamw_encode_polar": (_i32, [_p, _i32, _i64, _i64, _i64, _p, _p, _i32, _u64, _p, _i32, _p, _i32, _p, _p, _p,
                                 _sz, _p]),
    "qamw_channel_rms_workspace_bytes": (_sz, [_i64, _i64]),
    "qamw_channel_rms": (_i32, [_p, _i32, _i64, _i64, _i64, _p, _p, _sz, _p]),
    "qamw_output_error_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "qamw_output_error": (_i32, [_p, _i32, _i64, _i64, _i64, _p, _i32, _i64, _i64, _p, _i32, _i64, _p, _p, _sz,
                                 _p]),
    "qamw_rotate_activations": (_i32, [_p, _i32, _i64, _i64, _i64, _p, _i32, _u64, _p, _i64, _p]),
    "qamw_decode_matmul": (_i32, [_p, _i64, _i64, _i64, _p, _p, _i64, _p, _p, _i32, _p, _i32, _i64, _p]),
    "qamw_decode": (_i32, [_p, _p, _i64, _i64, _p, _p, _i32, _u64, _p, _i32, _p, _i32, _i64, _p]),
}

_LIB = None


class QamwError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed with status {status}: {message}")
        self.status = status


def load(path: str = ""):
    """Load libqamw.so once and attach the prototypes.  The path defaults to
    the in-tree build; the environment variable QAMW_LIBRARY can name another
    build of the same sources (for instance the host-sanitized one)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = path or os.environ.get("QAMW_LIBRARY") or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first (python -m vector_codebook_codec_amd._build "
                           "or __graft_entry__.build())")
    lib = _c.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def check(fn: str, status: int) -> None:
    if status != QAMW_OK:
        raise QamwError(fn, status, load().qamw_last_error().decode())
