"""ctypes declarations of the C ABI in include/sg.h (argument marshalling only)."""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsg.so")

SG_OK, SG_ERR_INVALID_ARG, SG_ERR_UNSUPPORTED, SG_ERR_WEIGHTS, SG_ERR_WORKSPACE, SG_ERR_HIP = 0, -1, -2, -3, -4, -5
SG_F32, SG_BF16 = 0, 1
SG_HEAD_SINKHORN, SG_HEAD_DOUBLE_SOFTMAX = 0, 1
SG_CROSS_STANDARD, SG_CROSS_BIDIRECTIONAL = 0, 1
SG_MAX_ENC = 8
SG_MAX_BATCH = 64
SG_N_STAGE_EVENTS = 6
SG_K_NONE, SG_K_GEMM, SG_K_ATTENTION, SG_K_SINKHORN = 0, 1, 2, 3
SG_FLAG_NO_GRAPH = 1
SG_FLAG_SINKHORN_TWO_SWEEP = 2
SG_FLAG_SINKHORN_ONE_SWEEP = 4
SG_FLAG_EARLY_EXIT = 8
SG_FLAG_PRUNE = 16
SG_FLAG_SHARED_SIMILARITY = 32

STATUS_NAMES = {0: "SG_OK", -1: "SG_ERR_INVALID_ARG", -2: "SG_ERR_UNSUPPORTED", -3: "SG_ERR_WEIGHTS",
                -4: "SG_ERR_WORKSPACE", -5: "SG_ERR_HIP"}


class SgWeights(C.Structure):
    _fields_ = [("D", C.c_int32), ("H", C.c_int32), ("n_enc", C.c_int32),
                ("enc", C.c_int32 * SG_MAX_ENC), ("L_max", C.c_int32), ("dtype", C.c_int32),
                ("head", C.c_int32), ("cross", C.c_int32), ("rope", C.c_int32), ("adaptive", C.c_int32),
                ("blob", C.c_void_p), ("blob_bytes", C.c_size_t)]


class SgOpts(C.Structure):
    _fields_ = [("stream", C.c_void_p), ("workspace", C.c_void_p), ("workspace_bytes", C.c_size_t),
                ("match_threshold", C.c_float), ("image_size", C.c_float * 4),
                ("out_matches1", C.c_void_p), ("out_scores1", C.c_void_p),
                ("out_desc_A", C.c_void_p), ("out_desc_B", C.c_void_p),
                ("out_logP", C.c_void_p), ("logP_ld", C.c_int64),
                ("stage_events", C.c_void_p), ("n_stage_events", C.c_int32),
                ("timed_kernel", C.c_int32), ("kernel_events", C.c_void_p),
                ("n_kernel_events", C.c_int32), ("n_kernel_launches", C.POINTER(C.c_int32)),
                ("flags", C.c_int32), ("depth_confidence", C.c_float), ("width_confidence", C.c_float),
                ("prune_min_points", C.c_int32), ("out_exit_layer", C.POINTER(C.c_int32)),
                ("out_prune0", C.c_void_p), ("out_prune1", C.c_void_p)]


_P = C.c_void_p
_I = C.c_int32
_F = C.c_float
_W = C.POINTER(SgWeights)
_O = C.POINTER(SgOpts)

SIGNATURES = {
    "sg_weights_count": (_I, [_W]),
    "sg_weights_tensor": (_I, [_W, _I, C.POINTER(C.c_size_t), C.POINTER(_I), C.POINTER(_I)]),
    "sg_weights_bytes": (C.c_size_t, [_W]),
    "sg_workspace_size": (C.c_size_t, [_W, _I, _I, _I]),
    "sg_match": (_I, [_P, _P, _P, _I, _P, _P, _P, _I, _W, _I, _I, _P, _P, _O]),
    "sg_match_batch": (_I, [_I, _I, _I, C.POINTER(_I), C.POINTER(_I), _P, _P, _P, _P, _P, _P, _W, _I, _I,
                            _P, _P, _O]),
    "sg_stage_encode": (_I, [_P, _P, _P, _I, _F, _F, _W, _P, _O]),
    "sg_stage_gnn": (_I, [_P, _I, _P, _I, _W, _I, _I, _O]),
    "sg_stage_gnn_pos": (_I, [_P, _P, _I, _P, _P, _I, _W, _I, _I, _O]),
    "sg_stage_project": (_I, [_P, _I, _W, _P, _O]),
    "sg_stage_scores": (_I, [_P, _I, _P, _I, _W, _P, C.c_int64, _O]),
    "sg_stage_scores_workspace_size": (C.c_size_t, [_I, _I, _I]),
    "sg_stage_match": (_I, [_P, _I, _P, _I, _I, _F, _I, _P, _P, _O]),
    "sg_stage_match_workspace_size": (C.c_size_t, [_I, _I, _I]),
    "sg_stage_match_ds": (_I, [_P, _P, _I, _P, _P, _I, _I, _P, _F, _P, _P, _O]),
    "sg_stage_match_ds_workspace_size": (C.c_size_t, [_I, _I, _I]),
    "sg_stage_sinkhorn": (_I, [_P, C.c_int64, _I, _I, _I, _P, _P, _P, C.c_int64, _O]),
    "sg_stage_sinkhorn_workspace_size": (C.c_size_t, [_I, _I]),
    "sg_stage_sinkhorn_noalloc": (_I, [_P, C.c_int64, _I, _I, _I, _P, _P, _P, C.c_int64, _P]),
    "sg_stage_extract": (_I, [_P, C.c_int64, _I, _I, _F, _P, _P, _P, _P, _O]),
    "sg_last_error": (C.c_char_p, []),
    "sg_version": (C.c_char_p, []),
}

_lib = None


def load():
    """Load the in-tree libsg.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                               "(python -m learned_sparse_feature_amd.build)")
        lib = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class SgError(RuntimeError):
    def __init__(self, status, fn):
        msg = load().sg_last_error().decode(errors="replace")
        super().__init__(f"{fn} -> {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def check(status, fn):
    if status != SG_OK:
        raise SgError(status, fn)
