"""ctypes mirror of include/attn_bwd.h and the library loader.

The loader never builds: if libattn_bwd.so is missing, every entry point raises
(no CPU fallback exists).  Build it with ``python -m scaled_dot_product_bwd_amd.build``
or ``__graft_entry__.build()``.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))

ATTN_F32, ATTN_BF16 = 0, 1
ATTN_WRT_Q, ATTN_WRT_K, ATTN_WRT_V, ATTN_WRT_ALL = 0, 1, 2, 3
ATTN_MASK_NONE, ATTN_MASK_CAUSAL, ATTN_MASK_KEYPAD, ATTN_MASK_WINDOW, ATTN_MASK_BIAS = 0, 1, 2, 3, 4
ATTN_MASK_FLAG_CAUSAL = 0x1
ATTN_OK, ATTN_E_INVALID, ATTN_E_UNSUPPORTED, ATTN_E_WORKSPACE, ATTN_E_HIP = 0, -1, -2, -3, -4

STATUS_NAMES = {ATTN_E_INVALID: "ATTN_E_INVALID", ATTN_E_UNSUPPORTED: "ATTN_E_UNSUPPORTED",
                ATTN_E_WORKSPACE: "ATTN_E_WORKSPACE", ATTN_E_HIP: "ATTN_E_HIP"}

# Every symbol include/attn_bwd.h declares.
EXPORTED = ["attn_bwd_workspace_bytes", "attn_bwd", "attn_bwd_row_stats", "attn_bwd_kv",
            "attn_bwd_dq", "attn_bwd_stats_dq", "attn_bwd_paged_plan_words", "attn_bwd_paged_plan_build",
            "attn_bwd_paged", "attn_bwd_paged_row_stats", "attn_bwd_paged_dq",
            "attn_bwd_from_forward", "attn_bwd_paged_q_workspace_bytes",
            "attn_bwd_last_error", "attn_bwd_noalloc", "attn_bwd_paged_stats_dq",
            "attn_bwd_split_workspace_bytes"]

# Plan header words (scaled_dot_product_bwd_amd/csrc/paged.hpp).
PLAN_MAGIC = 0x32504241
PLAN_ITEM_SLOTS = 128
# Link record words (LI_* in paged.hpp).
(LI_MIN_TOK, LI_MAX_TOK, LI_ALL_VALID, LI_QH0, LI_NQH, LI_MINPOS, LI_MAXPOS, LI_SEQ) = range(8)
LINK_INFO_WORDS = 8
(W_MAGIC, W_WORDS, W_NSEQ, W_NQ, W_HEADS, W_KV_HEADS, W_PAGE_SIZE, W_POOL_PAGES, W_ITEMS,
 W_LINKS, W_QH, W_LISTED, W_OFF_ITEM_LINKS, W_OFF_ITEM_SLOTS, W_OFF_LINK_SEQ, W_OFF_LINK_INFO,
 W_OFF_LINK_TOK, W_OFF_SEQ_QH, W_OFF_QH_RH, W_OFF_QH_POS, W_OFF_SEQ_MAXPOS,
 W_OFF_LISTED, W_OFF_SEQ_MINPOS, W_OFF_SEQ_TOK, W_OFF_TOK_SLOT, W_TOKENS, W_OFF_QBLK,
 W_QBLK, W_OFF_QPIECE, W_OFF_QBLK_PIECE, W_OFF_QPIECE_ORDER, W_QPIECES) = range(32)
PLAN_QPIECE_TOKENS = 1024


class AttnError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {message}")
        self.code = code


_i64x3 = ctypes.c_int64 * 3
_i64x4 = ctypes.c_int64 * 4


class AttnBwdArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("wrt", ctypes.c_int32),
        ("B", ctypes.c_int64), ("H", ctypes.c_int64), ("Sq", ctypes.c_int64),
        ("Sk", ctypes.c_int64), ("D", ctypes.c_int64),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("dy", ctypes.c_void_p),
        ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
        ("q_stride", _i64x3), ("k_stride", _i64x3), ("v_stride", _i64x3), ("dy_stride", _i64x3),
        ("dq_stride", _i64x3), ("dk_stride", _i64x3), ("dv_stride", _i64x3),
        ("mask_kind", ctypes.c_int32), ("mask_flags", ctypes.c_int32),
        ("window", ctypes.c_int64),
        ("mask", ctypes.c_void_p), ("mask_stride", _i64x4),
        ("mask_threshold", ctypes.c_float), ("scale", ctypes.c_float),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("Hkv", ctypes.c_int64),
    ]


class AttnBwdPagedArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("need", ctypes.c_int32),
        ("heads", ctypes.c_int32), ("kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("causal", ctypes.c_int32),
        ("nq", ctypes.c_int32), ("pool_pages", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("q", ctypes.c_void_p), ("dy", ctypes.c_void_p),
        ("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
        ("stats", ctypes.c_void_p),
        ("plan_host", ctypes.c_void_p), ("plan", ctypes.c_void_p),
        ("dk_pool", ctypes.c_void_p), ("dv_pool", ctypes.c_void_p),
        ("mla", ctypes.c_int32), ("position_dim", ctypes.c_int32),
        ("qp", ctypes.c_void_p), ("kp_pool", ctypes.c_void_p),
        ("dkp_pool", ctypes.c_void_p),
        ("q_workspace", ctypes.c_void_p), ("q_workspace_bytes", ctypes.c_size_t),
        ("kv_workgroups", ctypes.c_int32), ("q_form", ctypes.c_int32),
    ]


_lib = None


def library_path() -> str:
    return os.path.join(HERE, "libattn_bwd.so")


def load_library():
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m scaled_dot_product_bwd_amd.build` "
                           "(the HIP library is required, there is no fallback)")
    lib = ctypes.CDLL(path)
    lib.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_bwd_workspace_bytes.argtypes = [ctypes.c_int64] * 3
    lib.attn_bwd_split_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_bwd_split_workspace_bytes.argtypes = [ctypes.c_int64] * 5
    for name in ("attn_bwd", "attn_bwd_row_stats", "attn_bwd_kv", "attn_bwd_dq",
                 "attn_bwd_stats_dq", "attn_bwd_noalloc"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.POINTER(AttnBwdArgs), ctypes.c_void_p]
    _i32, _p = ctypes.c_int32, ctypes.c_void_p
    lib.attn_bwd_paged_plan_words.restype = ctypes.c_int64
    lib.attn_bwd_paged_plan_words.argtypes = [_i32, _p, _i32, _i32, _i32, _i32, _i32, _i32]
    lib.attn_bwd_paged_plan_build.restype = ctypes.c_int
    lib.attn_bwd_paged_plan_build.argtypes = [_i32, _p, _p, _i32, _i32, _p, _p, _i32, _i32, _i32,
                                              _i32, _p, ctypes.c_int64]
    lib.attn_bwd_paged.restype = ctypes.c_int
    lib.attn_bwd_paged.argtypes = [ctypes.POINTER(AttnBwdPagedArgs), ctypes.c_void_p]
    lib.attn_bwd_from_forward.restype = ctypes.c_int
    lib.attn_bwd_from_forward.argtypes = [ctypes.POINTER(AttnBwdArgs), ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64),
                                          ctypes.c_void_p]
    for name in ("attn_bwd_paged_row_stats", "attn_bwd_paged_dq"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.POINTER(AttnBwdPagedArgs), ctypes.c_void_p, ctypes.c_void_p]
    lib.attn_bwd_paged_stats_dq.restype = ctypes.c_int
    lib.attn_bwd_paged_stats_dq.argtypes = [ctypes.POINTER(AttnBwdPagedArgs), ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p]
    lib.attn_bwd_paged_q_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_bwd_paged_q_workspace_bytes.argtypes = [_p, _i32]
    lib.attn_bwd_last_error.restype = ctypes.c_char_p
    lib.attn_bwd_last_error.argtypes = []
    _lib = lib
    return lib
