"""ctypes signatures of libtsa's C ABI (include/tsa.h), declared on a loaded
library.  Kept apart from the package so that host-only checks can declare them
on another build of the library without importing torch."""
import ctypes


def declare_signatures(lib) -> None:
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.tsa_version.restype = ctypes.c_int
    lib.tsa_version.argtypes = []
    lib.tsa_last_error.restype = ctypes.c_char_p
    lib.tsa_last_error.argtypes = []
    lib.tsa_schedule_max_nnz.restype = i64
    lib.tsa_schedule_max_nnz.argtypes = [i64, i32, i32, i32]
    lib.tsa_build_schedule_workspace_bytes.restype = sz
    lib.tsa_build_schedule_workspace_bytes.argtypes = [i64, i64, i32]
    lib.tsa_build_schedule.restype = ctypes.c_int
    lib.tsa_build_schedule.argtypes = [
        vp, i32, i64, i64, i32, i32, i32, i32, vp, vp, i64, vp, vp, sz, ctypes.POINTER(i64), vp
    ]
    lib.tsa_build_schedule_ex.restype = ctypes.c_int
    lib.tsa_build_schedule_ex.argtypes = [
        vp, i32, i64, i64, i32, i32, i32, i32, i32, vp, vp, i64, vp, vp, sz, ctypes.POINTER(i64), vp
    ]
    lib.tsa_build_schedule_noalloc.restype = ctypes.c_int
    lib.tsa_build_schedule_noalloc.argtypes = [vp, i32, i64, i64, i32, i32, i32, i32, i32, vp, vp, i64, vp, vp]
    lib.tsa_dense_causal_schedule.restype = ctypes.c_int
    lib.tsa_dense_causal_schedule.argtypes = [i64, vp, vp, i64, vp]
    lib.tsa_segment_schedule_nnz.restype = i64
    lib.tsa_segment_schedule_nnz.argtypes = [i64, i32]
    lib.tsa_segment_schedule.restype = ctypes.c_int
    lib.tsa_segment_schedule.argtypes = [i64, i32, vp, vp, i64, vp]
    lib.tsa_scheduled_attention_fwd.restype = ctypes.c_int
    lib.tsa_scheduled_attention_fwd.argtypes = [
        vp, vp, vp, vp, i32, i64, i64, i64, i64, vp, vp, i64, i32, ctypes.c_float, vp
    ]
    lib.tsa_scheduled_attention_fwd_lse.restype = ctypes.c_int
    lib.tsa_scheduled_attention_fwd_lse.argtypes = [
        vp, vp, vp, vp, vp, i32, i64, i64, i64, i64, vp, vp, i64, i32, ctypes.c_float, vp
    ]
    lib.tsa_refine_schedule_max_nnz.restype = i64
    lib.tsa_refine_schedule_max_nnz.argtypes = [i64, i32, i64]
    lib.tsa_refine_schedule.restype = ctypes.c_int
    lib.tsa_refine_schedule.argtypes = [i64, i32, vp, vp, i64, vp, vp, i64, ctypes.POINTER(i64), vp]
    lib.tsa_schedule_transpose_workspace_bytes.restype = sz
    lib.tsa_schedule_transpose_workspace_bytes.argtypes = [i64]
    lib.tsa_schedule_transpose.restype = ctypes.c_int
    lib.tsa_schedule_transpose.argtypes = [i64, vp, vp, i64, vp, vp, i64, vp, sz, ctypes.POINTER(i64), vp]
    lib.tsa_scheduled_attention_bwd_workspace_bytes.restype = sz
    lib.tsa_scheduled_attention_bwd_workspace_bytes.argtypes = [i64, i64, i64]
    lib.tsa_scheduled_attention_bwd.restype = ctypes.c_int
    lib.tsa_scheduled_attention_bwd.argtypes = [
        vp, vp, vp, vp, vp, vp, i32, i64, i64, i64, i64, vp, vp, i64, vp, vp, i64, i32, ctypes.c_float,
        vp, vp, vp, vp, sz, vp,
    ]
