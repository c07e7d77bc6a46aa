"""ctypes declarations of libmpcg.so (the C ABI in include/mpcg.h).

Loading fails with an ImportError when the library has not been built; there
is no fallback implementation.
"""

from __future__ import annotations

import ctypes as ct
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmpcg.so")

CG_OK, CG_NOT_CONVERGED, CG_BREAKDOWN = 0, 1, 2
CG_EINVAL, CG_ENOMEM, CG_EDEVICE, CG_EINTERNAL = -1, -2, -3, -4
CG_FP64, CG_FP32, CG_BF16 = 0, 1, 2
CG_P1_ROUND_VECTOR, CG_P1_COLUMN_SCALE, CG_P1_PAD_COLUMNS = 1, 2, 4

i32, i64, f64, u8p = ct.c_int32, ct.c_int64, ct.c_double, ct.POINTER(ct.c_uint8)
vp = ct.c_void_p


class cg_tilecsc_view(ct.Structure):
    _fields_ = [
        ("n", i64), ("T", i64), ("nnz", i64), ("R", i32), ("C", i32),
        ("tile_row_ptr", ct.POINTER(i64)), ("tile_col_idx", ct.POINTER(i32)),
        ("tile_nnz_ptr", ct.POINTER(i64)), ("row_idx", ct.POINTER(ct.c_uint16)), ("col_local", u8p),
        ("val", ct.POINTER(f64)),
    ]


class cg_options(ct.Structure):
    _fields_ = [("jacobi", i32), ("window", i32), ("use_graph", i32), ("p1", i32), ("col_slices", i32),
                ("single_block", i32), ("stage_x", i32), ("reserved", i32 * 1)]


# name -> (restype, argtypes)
SIGNATURES = {
    "cg_tilecsc_from_csr": (ct.c_int, [i64, vp, vp, vp, i32, i32, ct.POINTER(vp)]),
    "cg_tilecsc_get_view": (ct.c_int, [vp, ct.POINTER(cg_tilecsc_view)]),
    "cg_tilecsc_col_ptr": (ct.c_int, [vp, vp]),
    "cg_tilecsc_perm": (ct.c_int, [vp, vp]),
    "cg_tilecsc_free": (None, [vp]),
    "cg_create": (ct.c_int, [vp, vp, ct.POINTER(cg_options), vp, ct.POINTER(vp)]),
    "cg_destroy": (ct.c_int, [vp]),
    "cg_set_precision_map": (ct.c_int, [vp, vp, i32]),
    "cg_get_active_map": (ct.c_int, [vp, vp]),
    "cg_map_from_magnitude": (ct.c_int, [vp, f64, f64]),
    "cg_record_window_maps": (ct.c_int, [vp, i32]),
    "cg_get_window_maps": (ct.c_int, [vp, i32, vp]),
    "cg_set_schedule_residual": (ct.c_int, [vp, i32, vp, vp]),
    "cg_set_schedule_tile_rule": (ct.c_int, [vp, i32, vp, f64, f64]),
    "cg_eval_tile_rule": (ct.c_int, [vp, f64]),
    "cg_set_schedule_pmag": (ct.c_int, [vp, f64, f64, i32]),
    "cg_record_column_codes": (ct.c_int, [vp, i32]),
    "cg_get_column_codes": (ct.c_int, [vp, i32, vp]),
    "cg_select_reuse_interval": (ct.c_int, [vp, i32, ct.c_int64, f64, vp, i32, vp, vp]),
    "cg_clear_schedule": (ct.c_int, [vp]),
    "cg_spmv": (ct.c_int, [vp, vp, vp, vp]),
    "cg_solve": (ct.c_int, [vp, vp, vp, f64, i32, vp, ct.POINTER(i32), vp, vp]),
    "cg_true_residual": (ct.c_int, [vp, vp, vp, ct.POINTER(f64), vp]),
    "cg_true_residual_noalloc": (ct.c_int, [vp, vp, vp, vp, vp]),
    "cg_stream_read": (ct.c_int, [vp, i64, vp, i32, vp]),
    "cg_stream_copy": (ct.c_int, [vp, vp, i64, i32, vp]),
    "cg_stream_mix": (ct.c_int, [vp, i64, vp, i64, vp, i32, vp]),
    "cg_get_map_trace": (ct.c_int, [vp, i32, vp, vp]),
    "cg_export_layout": (ct.c_int, [vp, vp, vp, vp, vp, vp, vp, vp, vp]),
    "cg_export_column_scale": (ct.c_int, [vp, vp]),
    "cg_tune_row_height": (ct.c_int, [i64, vp, vp, i32, i32, i64, vp, i32, vp, vp, vp, vp, vp, vp]),
    "cg_get_options": (ct.c_int, [vp, ct.POINTER(cg_options)]),
    "cg_get_sizes": (ct.c_int, [vp, ct.POINTER(i64), ct.POINTER(i64), ct.POINTER(i64),
                                ct.POINTER(i32), ct.POINTER(i32)]),
    "cg_device_bytes": (i64, [vp]),
    "cg_last_error": (ct.c_char_p, []),
    "cg_version": (ct.c_int, []),
}

_lib = None


def load() -> ct.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m mixed_precision_sparse_amd.build` (there is no fallback)")
    lib = ct.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class CGError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


def check(code: int) -> int:
    if code < 0:
        raise CGError(code, load().cg_last_error().decode(errors="replace"))
    return code
