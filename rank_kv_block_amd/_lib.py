"""ctypes declarations of libpred.so, the predictor's C ABI (see include/pred.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation behind these names.
"""

import ctypes
import os

# PRED_LIBRARY selects another build of the same library (e.g. the host-side
# sanitizer build the CPU tests load); by default the in-tree libpred.so.
LIB_PATH = os.environ.get("PRED_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpred.so")

PRED_OK = 0
PRED_ERR_INVALID_DIMS = -1
PRED_ERR_OUT_OF_RANGE = -2
PRED_ERR_OOM = -3
PRED_ERR_UNSUPPORTED = -4
PRED_ERR_NULL_ARG = -5
PRED_ERR_HIP = -6
PRED_ERR_WORKSPACE = -7
PRED_ERR_DEVICE = -8

PRED_FLAG_ZERO_AG = 1

PRED_NOALLOC_SCRATCH_BYTES = 8 << 20

PRED_SCORE_PATH_AUTO = 0
PRED_SCORE_PATH_DECODE = 1
PRED_SCORE_PATH_GENERIC = 2

ERROR_NAMES = {
    PRED_ERR_INVALID_DIMS: "INVALID_DIMS",
    PRED_ERR_OUT_OF_RANGE: "OUT_OF_RANGE",
    PRED_ERR_OOM: "OOM",
    PRED_ERR_UNSUPPORTED: "UNSUPPORTED",
    PRED_ERR_NULL_ARG: "NULL_ARG",
    PRED_ERR_HIP: "HIP",
    PRED_ERR_WORKSPACE: "WORKSPACE",
    PRED_ERR_DEVICE: "DEVICE",
}


class PredDims(ctypes.Structure):
    _fields_ = [
        ("num_layers", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("r", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_blocks", ctypes.c_int64),
    ]


_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_u64 = ctypes.c_uint64
_PD = ctypes.POINTER(PredDims)

# name -> (restype, argtypes)
SIGNATURES = {
    "pred_a_g_bytes": (_i64, [_PD]),
    "pred_check_fit": (ctypes.c_int, [_PD, _u64]),
    "pred_limits": (ctypes.c_char_p, []),
    "pred_create": (ctypes.c_int, [_PD, _u64, ctypes.c_uint32, _vp, ctypes.POINTER(_vp)]),
    "pred_create_with_projection": (ctypes.c_int, [_PD, _vp, ctypes.c_uint32, _vp, ctypes.POINTER(_vp)]),
    "pred_destroy": (None, [_vp]),
    "pred_project_q": (ctypes.c_int, [_vp, _vp, _i64, _vp, _vp]),
    "pred_project_kv_block": (ctypes.c_int, [_vp, _i32, _i32, _vp, _vp, _i64, _vp]),
    "pred_project_step": (ctypes.c_int, [_vp, _i32, _i32, _vp, _vp, _i64, _vp, _i64, _vp, _vp]),
    "pred_score_blocks": (ctypes.c_int, [_vp, _i32, _i32, _vp, _i32, _vp, _i64, _i32, _vp, _vp]),
    "pred_score_blocks_masked": (ctypes.c_int, [_vp, _i32, _i32, _vp, _i32, _vp, _i64, _i32, _vp, _vp, _vp]),
    "pred_rank_victims": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp, _vp, ctypes.c_size_t, _vp]),
    "pred_rank_victims_noalloc": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp, _vp]),
    "pred_select_victims": (ctypes.c_int, [_vp, _vp, _i64, _i64, _i64, _vp, _vp, ctypes.c_size_t, _vp]),
    "pred_score_kernel_name": (ctypes.c_char_p, [_vp, _i32]),
    "pred_score_kernel_variant": (ctypes.c_char_p, [_vp, _i32, _i64]),
    "pred_set_score_path": (ctypes.c_int, [_i32]),
    "pred_get_score_path": (ctypes.c_int, []),
    "pred_score_rows": (ctypes.c_int, [_vp, _i32, _vp, _i64, _i64, _vp, _i64, _vp, _i64, _vp]),
    "pred_select_keep": (ctypes.c_int, [_vp, _vp, _i64, _i64, _i64, _i32, _i64, _vp, _vp, ctypes.c_size_t, _vp]),
    "pred_decode_step": (ctypes.c_int, [_vp, _i32, _i32, _vp, _vp, _i64, _vp, _i32, _vp, _vp, _i64, _i32, _vp,
                                         _vp, _i64, _vp, _vp, ctypes.c_size_t, _vp]),
    "pred_rank_workspace_bytes": (ctypes.c_size_t, [_i64, _i64]),
    "pred_projection_host": (ctypes.c_int, [_i32, _i32, _u64, _vp]),
    "pred_copy_projection": (ctypes.c_int, [_vp, _vp]),
    "pred_a_g_ptr": (_vp, [_vp]),
    "pred_read_slot": (ctypes.c_int, [_vp, _i32, _i64, _vp, _vp]),
    "pred_get_dims": (ctypes.c_int, [_vp, _PD]),
    "pred_device_error": (ctypes.c_int, [_vp, _vp]),
    "pred_last_error": (ctypes.c_char_p, []),
    "pred_version": (ctypes.c_char_p, []),
}

_LIB = None


def load():
    """Load libpred.so once and declare its signatures; raise if it is missing."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built: run `python -c 'import __graft_entry__ as g; g.build()'` "
            "(hipcc --offload-arch=gfx950) first")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib
