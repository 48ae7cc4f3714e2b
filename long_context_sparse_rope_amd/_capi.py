"""ctypes declarations of liblcsr.so (include/lcsr.h)."""

import ctypes
import os

from . import build as _build

LCSR_OK = 0
LCSR_EINVAL = -1
LCSR_ENOTSUP = -2
LCSR_EWORKSPACE = -3
LCSR_EHIP = -4

LCSR_BF16 = 0
LCSR_FP32 = 1
LCSR_FP16 = 2

LCSR_ROPE_YARN_FREQ = 0x1
LCSR_ROPE_NO_ROTATE = 0x2
LCSR_ROPE_OUT_FP16 = 0x4
LCSR_EST_SELECT_ONLY = 0x1
LCSR_ATTN_DENSE = 0x1
LCSR_BS_SELECT_ONLY = 0x1

LCSR_WS_ESTIMATE = 0
LCSR_WS_ATTN = 1
LCSR_WS_RECALL = 2
LCSR_WS_DECODE = 3
LCSR_WS_BLOCK_EST = 4
LCSR_WS_BLOCK_ATTN = 5

EXPORTED = ("lcsr_workspace_bytes", "lcsr_last_error", "lcsr_softmax_scale",
            "lcsr_rope_yarn_apply",
            "lcsr_dca_positions", "lcsr_vs_pattern_estimate",
            "lcsr_vs_sparse_attn_prefill", "lcsr_attn_decode", "lcsr_attn_decode_noalloc",
            "lcsr_attn_recall_check",
            "lcsr_pattern_fill_a_shape", "lcsr_block_sparse_estimate",
            "lcsr_block_sparse_attn_prefill", "lcsr_block_sparse_recall_check")


class lcsr_rope_t(ctypes.Structure):
    _fields_ = [("base", ctypes.c_double), ("yarn_factor", ctypes.c_double),
                ("orig_max_pos", ctypes.c_int64), ("beta_fast", ctypes.c_double),
                ("beta_slow", ctypes.c_double), ("flags", ctypes.c_uint32)]


class lcsr_dca_t(ctypes.Structure):
    _fields_ = [("chunk", ctypes.c_int64), ("local", ctypes.c_int64)]


class lcsr_problem_t(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("q_dtype", ctypes.c_int32),
                ("q_stride_h", ctypes.c_int64), ("q_stride_t", ctypes.c_int64),
                ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
                ("kv_stride_h", ctypes.c_int64), ("kv_stride_t", ctypes.c_int64),
                ("n_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("chunk_start", ctypes.c_int64),
                ("chunk_len", ctypes.c_int64), ("rope", lcsr_rope_t),
                ("dca", lcsr_dca_t), ("sm_scale", ctypes.c_float)]


class lcsr_pattern_t(ctypes.Structure):
    _fields_ = [("vert_idx", ctypes.c_void_p), ("vert_cnt", ctypes.c_void_p),
                ("max_vert", ctypes.c_int32), ("slash_idx", ctypes.c_void_p),
                ("slash_cnt", ctypes.c_void_p), ("max_slash", ctypes.c_int32)]


_lib = None


def library_path():
    return _build.LIB


def load():
    """Load liblcsr.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first "
                           "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    vp, i32, i64, u32, f32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                              ctypes.c_uint32, ctypes.c_float)
    lib.lcsr_workspace_bytes.restype = ctypes.c_size_t
    lib.lcsr_workspace_bytes.argtypes = [ctypes.c_int, P(lcsr_problem_t), i32, i32]
    lib.lcsr_last_error.restype = ctypes.c_char_p
    lib.lcsr_last_error.argtypes = []
    lib.lcsr_softmax_scale.restype = ctypes.c_float
    lib.lcsr_softmax_scale.argtypes = [P(lcsr_rope_t), i32]
    lib.lcsr_rope_yarn_apply.restype = ctypes.c_int
    lib.lcsr_rope_yarn_apply.argtypes = [vp, i32, i64, i64, vp, i64, i64, i64, i64, i64, vp,
                                         P(lcsr_rope_t), f32, u32, vp]
    lib.lcsr_dca_positions.restype = ctypes.c_int
    lib.lcsr_dca_positions.argtypes = [i64, i64, P(lcsr_dca_t), vp, vp, vp, vp, vp]
    lib.lcsr_block_sparse_estimate.restype = ctypes.c_int
    lib.lcsr_block_sparse_estimate.argtypes = [P(lcsr_problem_t), vp, vp, i32, vp, vp, vp, u32,
                                               vp, ctypes.c_size_t, vp]
    lib.lcsr_block_sparse_attn_prefill.restype = ctypes.c_int
    lib.lcsr_block_sparse_attn_prefill.argtypes = [P(lcsr_problem_t), vp, vp, i32, vp, vp, i32,
                                                   i64, i64, vp, vp, vp, ctypes.c_size_t, vp]
    lib.lcsr_block_sparse_recall_check.restype = ctypes.c_int
    lib.lcsr_block_sparse_recall_check.argtypes = [P(lcsr_problem_t), vp, vp, i32, vp, vp, i32,
                                                   vp, vp, vp, vp]
    lib.lcsr_pattern_fill_a_shape.restype = ctypes.c_int
    lib.lcsr_pattern_fill_a_shape.argtypes = [P(lcsr_pattern_t), i32, vp, i32, i32, i64, vp]
    lib.lcsr_vs_pattern_estimate.restype = ctypes.c_int
    lib.lcsr_vs_pattern_estimate.argtypes = [P(lcsr_problem_t), i32, vp, vp, vp,
                                             P(lcsr_pattern_t), vp, vp, u32, vp,
                                             ctypes.c_size_t, vp]
    lib.lcsr_vs_sparse_attn_prefill.restype = ctypes.c_int
    lib.lcsr_vs_sparse_attn_prefill.argtypes = [P(lcsr_problem_t), P(lcsr_pattern_t), vp, vp,
                                                i32, i64, i64, vp, vp, u32, vp,
                                                ctypes.c_size_t, vp]
    lib.lcsr_attn_decode.restype = ctypes.c_int
    lib.lcsr_attn_decode.argtypes = [P(lcsr_problem_t), vp, i32, i64, i64, vp, vp,
                                     ctypes.c_size_t, vp]
    lib.lcsr_attn_decode_noalloc.restype = ctypes.c_int
    lib.lcsr_attn_decode_noalloc.argtypes = [P(lcsr_problem_t), vp, i32, i64, i64, vp, vp]
    lib.lcsr_attn_recall_check.restype = ctypes.c_int
    lib.lcsr_attn_recall_check.argtypes = [P(lcsr_problem_t), P(lcsr_pattern_t), vp, vp, i32,
                                           vp, vp, vp, vp, ctypes.c_size_t, vp]
    _lib = lib
    return lib
