"""ctypes declarations of the C ABI in include/fastocr.h."""

from __future__ import annotations

import ctypes
import os

c_int32, c_int64, c_double, c_float, c_void_p = (ctypes.c_int32, ctypes.c_int64, ctypes.c_double,
                                                 ctypes.c_float, ctypes.c_void_p)

OK = 0
ERR_INVALID_ARG = -1
ERR_STATE = -2
ERR_HIP = -3
ERR_OOM = -4
ERR_SCRATCH = -5
STATIC_SCRATCH_MIB = 64  # FASTOCR_STATIC_SCRATCH_MIB

DTYPE_F32 = 0
DTYPE_BF16 = 1
MODE_PRUNED = 0
MODE_FULL = 1

FLAG_LENS_CLAMPED = 1
FLAG_INDEX_CLAMPED = 2

KC_FULL_SPLIT = 0
KC_FOCAL_SPLIT = 1
KC_SPARSE_SPLIT = 2
KC_MERGE = 3
KC_TOPK = 4
KC_COUNT = 5
KC_NAMES = ("full_split", "focal_split", "sparse_split", "merge", "topk")


class Config(ctypes.Structure):
    _fields_ = [
        ("tau", c_double),
        ("sm_scale", c_float),
        ("num_layers", c_int32),
        ("num_q_heads", c_int32),
        ("num_kv_heads", c_int32),
        ("head_dim", c_int32),
        ("batch", c_int32),
        ("max_seq_len", c_int32),
        ("max_img_tokens", c_int32),
        ("min_img_tokens", c_int32),
        ("dtype", c_int32),
        ("num_focal", c_int32),
        ("warmup_steps", c_int32),
        ("mode", c_int32),
        ("max_text_tokens", c_int32),
        ("reprofile_every", c_int32),
    ]


class Info(ctypes.Structure):
    _fields_ = [
        ("step", c_int32),
        ("next_layer", c_int32),
        ("phase", c_int32),
        ("k_max", c_int32),
        ("full_rows_per_split", c_int32),
        ("full_max_splits", c_int32),
        ("sparse_rows_per_split", c_int32),
        ("sparse_max_splits", c_int32),
        ("sparse_direct", c_int32),
        ("focal_staged", c_int32),
        ("stream_rows", c_int32),
        ("profiles", c_int32),
        ("scratch_bytes", c_int64),
    ]


class Timing(ctypes.Structure):
    _fields_ = [("total_ms", c_double * KC_COUNT), ("launches", c_int64 * KC_COUNT),
                ("timed", c_int64 * KC_COUNT)]


LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfastocr.so")

# (name, restype, argtypes)
SIGNATURES = [
    ("fastocr_create", c_int32, [ctypes.POINTER(Config), c_void_p, ctypes.POINTER(c_void_p)]),
    ("fastocr_create_static", c_int32, [ctypes.POINTER(Config), c_void_p, ctypes.POINTER(c_void_p)]),
    ("fastocr_attend", c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    ("fastocr_attend_append", c_int32,
     [c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    ("fastocr_profile_warmup", c_int32, [c_void_p, ctypes.POINTER(c_int32)]),
    ("fastocr_get_focal_layers", c_int32, [c_void_p, ctypes.POINTER(c_int32)]),
    ("fastocr_destroy", c_int32, [c_void_p]),
    ("fastocr_get_status", c_int32, [c_void_p, ctypes.POINTER(c_int32)]),
    ("fastocr_get_selection", c_int32, [c_void_p, c_void_p, c_void_p]),
    ("fastocr_get_scores", c_int32, [c_void_p, c_void_p]),
    ("fastocr_get_layer_ratios", c_int32, [c_void_p, ctypes.POINTER(c_double)]),
    ("fastocr_set_focal_layers", c_int32, [c_void_p, ctypes.POINTER(c_int32), c_int32]),
    ("fastocr_set_selection", c_int32, [c_void_p, c_void_p, c_void_p]),
    ("fastocr_get_info", c_int32, [c_void_p, ctypes.POINTER(Info)]),
    ("fastocr_plan_launch", c_int32, [ctypes.POINTER(Config), c_int32, ctypes.POINTER(Info)]),
    ("fastocr_set_timing", c_int32, [c_void_p, c_int32]),
    ("fastocr_get_timing", c_int32, [c_void_p, ctypes.POINTER(Timing)]),
    ("fastocr_reset_timing", c_int32, [c_void_p]),
    ("fastocr_select_topk", c_int32, [c_void_p, c_int32, c_void_p, c_int32, c_double, c_void_p,
                                      c_int32, c_void_p, c_void_p]),
    ("fastocr_state_bytes", c_int32, [c_void_p, ctypes.POINTER(c_int64)]),
    ("fastocr_save_state", c_int32, [c_void_p, c_void_p, c_int64]),
    ("fastocr_load_state", c_int32, [c_void_p, c_void_p, c_int64]),
    ("fastocr_image_first_map", c_int32, [ctypes.POINTER(c_int32), c_int32, c_int32, ctypes.POINTER(c_int32)]),
    ("fastocr_pack_rows", c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32,
                                    c_int32, c_void_p, c_void_p]),
    ("fastocr_probe_read", c_int32, [c_void_p, c_int64, c_int32, c_void_p, c_void_p]),
    ("fastocr_kept_count", c_int32, [c_double, c_int32]),
    ("fastocr_choose_focal_layers", c_int32, [ctypes.POINTER(c_double), c_int32, c_int32,
                                              ctypes.POINTER(c_int32)]),
    ("fastocr_error_string", ctypes.c_char_p, [c_int32]),
]

_lib = None


def load() -> ctypes.CDLL:
    """Load the built HIP library; raise if it is missing (no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"HIP library not found at {LIB_PATH}; build it with "
                "`python -c 'import __graft_entry__ as g; g.build()'`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib
