"""ctypes view of libgdr.so (include/gdr.h).  Loading fails loudly if the
library has not been built: there is no fallback path."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgdr.so")

GDR_BF16, GDR_FP16, GDR_FP32 = 0, 1, 2

STATUS = {
    0: "GDR_OK", 1: "GDR_ERR_NULL", 2: "GDR_ERR_SHAPE", 3: "GDR_ERR_HEAD_DIM",
    4: "GDR_ERR_DTYPE", 5: "GDR_ERR_HEADS", 6: "GDR_ERR_VARLEN", 7: "GDR_ERR_WORKSPACE",
    8: "GDR_ERR_DEVICE", 9: "GDR_ERR_HIP", 10: "GDR_ERR_ARG",
}


class Problem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("T", ctypes.c_int32), ("Hq", ctypes.c_int32),
        ("Hv", ctypes.c_int32), ("K", ctypes.c_int32), ("V", ctypes.c_int32),
        ("N", ctypes.c_int32),
        ("cu_seqlens_dev", ctypes.c_void_p),
        ("cu_seqlens_host", ctypes.c_void_p),
        ("in_dtype", ctypes.c_int), ("g_dtype", ctypes.c_int),
        ("scale", ctypes.c_float),
        ("state_v_first", ctypes.c_int32),
        ("cp_segments", ctypes.c_int32),
        ("wave_tiles", ctypes.c_int32),
        ("use_qk_l2norm", ctypes.c_int32),
        ("beta_sigmoid", ctypes.c_int32),
        ("neg_eigval", ctypes.c_int32),
        ("use_gate", ctypes.c_int32),
        ("gate_A_log", ctypes.c_void_p),
        ("gate_dt_bias", ctypes.c_void_p),
        ("h_packed", ctypes.c_int32),
    ]


# every symbol include/gdr.h declares
EXPORTS = [
    "gdr_status_string", "gdr_last_error", "gdr_check_supported", "gdr_check_device",
    "gdr_chunk_fwd_workspace_size", "gdr_chunk_bwd_workspace_size", "gdr_chunk_fwd",
    "gdr_chunk_bwd", "gdr_prepare_lens_i32", "gdr_prepare_lens_i64",
    "gdr_prepare_chunk_indices_i32", "gdr_prepare_chunk_indices_i64",
    "gdr_prepare_chunk_offsets_i32", "gdr_prepare_chunk_offsets_i64",
    "gdr_prepare_chunk_token_starts_i64", "gdr_profile_enable", "gdr_profile_read",
    "gdr_plan_info", "gdr_recurrent_fwd", "gdr_chunk_bwd_gate", "gdr_chunk_fwd_noalloc",
    "gdr_chunk_bwd_states", "gdr_chunk_bwd_states_workspace_size", "gdr_chunk_fwd_states",
    "gdr_chunk_trans_size", "gdr_bwd_pipeline_info",
]


class GdrError(RuntimeError):
    def __init__(self, status: int, msg: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__("%s: %s" % (self.name, msg))


def _declare(lib):
    P = ctypes.c_void_p
    PP = ctypes.POINTER(Problem)
    I64 = ctypes.c_int64
    S = ctypes.c_size_t
    st = ctypes.c_int
    lib.gdr_status_string.argtypes = [st]
    lib.gdr_status_string.restype = ctypes.c_char_p
    lib.gdr_last_error.argtypes = []
    lib.gdr_last_error.restype = ctypes.c_char_p
    lib.gdr_check_supported.argtypes = [PP, ctypes.c_char_p, S]
    lib.gdr_check_supported.restype = st
    lib.gdr_check_device.argtypes = []
    lib.gdr_check_device.restype = st
    lib.gdr_chunk_fwd_workspace_size.argtypes = [PP]
    lib.gdr_chunk_fwd_workspace_size.restype = S
    lib.gdr_chunk_bwd_workspace_size.argtypes = [PP]
    lib.gdr_chunk_bwd_workspace_size.restype = S
    lib.gdr_chunk_fwd.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, P, P, S, P]
    lib.gdr_chunk_fwd.restype = st
    lib.gdr_chunk_bwd_states_workspace_size.argtypes = [PP]
    lib.gdr_chunk_bwd_states_workspace_size.restype = S
    lib.gdr_chunk_bwd_states.argtypes = [PP] + [P] * 12 + [S] + [P] * 9 + [S, P]
    lib.gdr_bwd_pipeline_info.argtypes = [PP, ctypes.POINTER(ctypes.c_int32),
                                          ctypes.POINTER(ctypes.c_int32), ctypes.c_int32]
    lib.gdr_bwd_pipeline_info.restype = st
    lib.gdr_chunk_trans_size.argtypes = [PP]
    lib.gdr_chunk_trans_size.restype = S
    lib.gdr_chunk_fwd_states.argtypes = [PP] + [P] * 11 + [S] + [P] * 2 + [S, P]
    lib.gdr_chunk_fwd_states.restype = st
    lib.gdr_chunk_bwd_states.restype = st
    lib.gdr_chunk_fwd_noalloc.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, P, P]
    lib.gdr_chunk_fwd_noalloc.restype = st
    lib.gdr_chunk_bwd.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, S, P]
    lib.gdr_chunk_bwd.restype = st
    lib.gdr_chunk_bwd_gate.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P,
                                       P, S, P]
    lib.gdr_chunk_bwd_gate.restype = st
    lib.gdr_recurrent_fwd.argtypes = [PP, P, P, P, P, P, P, P, P, P]
    lib.gdr_recurrent_fwd.restype = st
    for name in ("gdr_prepare_lens_i32", "gdr_prepare_lens_i64"):
        getattr(lib, name).argtypes = [P, I64, P]
        getattr(lib, name).restype = st
    for name in ("gdr_prepare_chunk_indices_i32", "gdr_prepare_chunk_indices_i64",
                 "gdr_prepare_chunk_offsets_i32", "gdr_prepare_chunk_offsets_i64",
                 "gdr_prepare_chunk_token_starts_i64"):
        getattr(lib, name).argtypes = [P, I64, I64, P, ctypes.POINTER(I64)]
        getattr(lib, name).restype = st


def _declare_profile(lib):
    lib.gdr_profile_enable.argtypes = [ctypes.c_int]
    lib.gdr_profile_enable.restype = ctypes.c_int
    lib.gdr_profile_read.argtypes = [ctypes.c_char_p, ctypes.c_size_t, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_int]
    lib.gdr_profile_read.restype = ctypes.c_int
    lib.gdr_plan_info.argtypes = [ctypes.POINTER(Problem), ctypes.c_int,
                                  ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
    lib.gdr_plan_info.restype = ctypes.c_int


def load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            "libgdr.so is not built (expected at %s); run gated_delta_rule_66_amd/build.py"
            % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    _declare(lib)
    _declare_profile(lib)
    return lib


lib = load()


def check(status: int):
    if status != 0:
        raise GdrError(status, lib.gdr_last_error().decode(errors="replace"))
