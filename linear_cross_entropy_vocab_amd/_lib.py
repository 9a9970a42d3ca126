"""ctypes loader for liblce.so and the raw C-ABI signatures (see include/lce.h)."""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblce.so")

LCE_OK = 0
STATUS_NAMES = {0: "LCE_OK", 1: "LCE_ERR_NULL", 2: "LCE_ERR_SHAPE", 3: "LCE_ERR_DTYPE",
                4: "LCE_ERR_ALIGNMENT", 5: "LCE_ERR_WORKSPACE", 6: "LCE_ERR_ARG",
                7: "LCE_ERR_TARGET_RANGE", 8: "LCE_ERR_HIP", 9: "LCE_ERR_SCRATCH_LIMIT"}
NOALLOC_MAX_ROWS = 262144
DTYPE_F32 = 0
DTYPE_BF16 = 1
DTYPE_F16 = 2
REDUCTION_MEAN = 0
REDUCTION_SUM = 1
FLAG_CHECK_TARGETS = 1
FLAG_GRAD_W_FP32 = 2
FLAG_SORT_VOCAB = 4
NUM_STAGES = 7

EXPORTS = ("lce_fwd_bwd", "lce_fwd_bwd_profiled", "lce_fwd_bwd_filtered", "lce_filter_tile_shape",
           "lce_fwd_bwd_workspace_bytes",
           "lce_fwd_bwd_chunked", "lce_fwd_bwd_chunked_workspace_bytes",
           "lce_rows_forward", "lce_rows_backward", "lce_rows_workspace_bytes",
           "lce_stage_name",
           "lce_ce_with_grad_inplace", "lce_ce_with_grad_inplace_noalloc", "lce_ce_workspace_bytes",
           "lce_stream_bandwidth", "lce_status_string", "lce_version")

_lib = None

c_vp = ctypes.c_void_p
c_i64 = ctypes.c_int64
c_f = ctypes.c_float


def load() -> ctypes.CDLL:
    """Load liblce.so (built in-tree by linear_cross_entropy_vocab_amd.build); raise if absent.

    LCE_LIBRARY, if set, names another build of the same library to load instead (the
    host-sanitizer build of build.build_host_sanitized)."""
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("LCE_LIBRARY") or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it first with "
            "`python -m linear_cross_entropy_vocab_amd.build` (there is no fallback path)")
    lib = ctypes.CDLL(path)
    fused = [c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, ctypes.c_int, c_i64, c_f, ctypes.c_int,
             ctypes.c_uint32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, ctypes.c_size_t, c_vp]
    lib.lce_fwd_bwd.argtypes = fused
    lib.lce_fwd_bwd.restype = ctypes.c_int
    lib.lce_fwd_bwd_profiled.argtypes = fused + [c_vp, c_vp]
    lib.lce_fwd_bwd_profiled.restype = ctypes.c_int
    lib.lce_fwd_bwd_filtered.argtypes = fused + [c_f, c_vp]
    lib.lce_fwd_bwd_filtered.restype = ctypes.c_int
    lib.lce_filter_tile_shape.argtypes = [c_i64, c_i64, c_i64, ctypes.c_int, c_vp, c_vp]
    lib.lce_filter_tile_shape.restype = ctypes.c_int
    lib.lce_fwd_bwd_workspace_bytes.argtypes = [c_i64, c_i64, c_i64, ctypes.c_int, ctypes.c_uint32]
    lib.lce_fwd_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.lce_fwd_bwd_chunked.argtypes = fused
    lib.lce_fwd_bwd_chunked.restype = ctypes.c_int
    lib.lce_fwd_bwd_chunked_workspace_bytes.argtypes = [c_i64, c_i64, c_i64, ctypes.c_int, ctypes.c_uint32]
    lib.lce_fwd_bwd_chunked_workspace_bytes.restype = ctypes.c_size_t
    lib.lce_rows_workspace_bytes.argtypes = [c_i64, c_i64, c_i64, ctypes.c_int, ctypes.c_uint32]
    lib.lce_rows_workspace_bytes.restype = ctypes.c_size_t
    rows_head = [c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, ctypes.c_int, c_i64, c_f, ctypes.c_uint32]
    lib.lce_rows_forward.argtypes = rows_head + [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, ctypes.c_size_t, c_vp]
    lib.lce_rows_forward.restype = ctypes.c_int
    lib.lce_rows_backward.argtypes = rows_head + [c_vp] * 9 + [ctypes.c_size_t, c_vp]
    lib.lce_rows_backward.restype = ctypes.c_int
    lib.lce_stage_name.argtypes = [ctypes.c_int]
    lib.lce_stage_name.restype = ctypes.c_char_p
    lib.lce_ce_with_grad_inplace.argtypes = [c_vp, c_vp, c_i64, c_i64, ctypes.c_int, c_i64, c_f, c_vp,
                                             c_vp, c_vp, c_vp, ctypes.c_size_t, c_vp]
    lib.lce_ce_with_grad_inplace.restype = ctypes.c_int
    lib.lce_ce_with_grad_inplace_noalloc.argtypes = [c_vp, c_vp, c_i64, c_i64, ctypes.c_int, c_i64, c_f, c_vp,
                                                     c_vp, c_vp, c_vp]
    lib.lce_ce_with_grad_inplace_noalloc.restype = ctypes.c_int
    lib.lce_stream_bandwidth.argtypes = [ctypes.c_int, c_vp, c_vp, ctypes.c_size_t, c_vp]
    lib.lce_stream_bandwidth.restype = ctypes.c_int
    lib.lce_ce_workspace_bytes.argtypes = [c_i64, c_i64, ctypes.c_int]
    lib.lce_ce_workspace_bytes.restype = ctypes.c_size_t
    lib.lce_status_string.argtypes = [ctypes.c_int]
    lib.lce_status_string.restype = ctypes.c_char_p
    lib.lce_version.argtypes = []
    lib.lce_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


class LCEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        lib = load()
        msg = lib.lce_status_string(status).decode()
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({msg})")


def check(status: int, where: str) -> None:
    if status != LCE_OK:
        raise LCEError(status, where)
