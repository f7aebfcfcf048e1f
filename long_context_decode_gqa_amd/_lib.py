"""ctypes view of the C ABI in include/attn_decode.h (libattn_decode.so)."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libattn_decode.so")

ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE_TOO_SMALL, ATTN_ERR_HIP = range(5)
ATTN_F32, ATTN_BF16, ATTN_I8 = 0, 1, 2
ATTN_QUANT_EXACT, ATTN_QUANT_ROW, ATTN_QUANT_STATIC = 0, 1, 2

vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t


class AttnKvGeom(ctypes.Structure):
    _fields_ = [("B", i32), ("KH", i32), ("D", i32), ("max_seq_len", i32),
                ("seq_lens", vp), ("seq_offset", vp), ("stride_h", i64), ("stride_t", i64),
                ("block_table", vp), ("page_tokens", i32), ("table_stride", i32), ("page_stride", i64)]


class AttnDecodeArgs(ctypes.Structure):
    _fields_ = [("kv", AttnKvGeom), ("G", i32), ("q_rows", i32), ("q_dtype", i32), ("kv_dtype", i32), ("out_dtype", i32),
                ("q", vp), ("k", vp), ("v", vp), ("k_scale", vp), ("k_part_tokens", i32), ("k_scale_stride", i32),
                ("v_scale", f32), ("q_quant", i32), ("q_scale", f32), ("token_idx", vp), ("n_idx", vp), ("idx_stride", i32), ("softmax_scale", f32),
                ("split_tokens", i32), ("workspace", vp), ("workspace_bytes", sz), ("out", vp), ("lse", vp),
                ("fixed_splits", i32)]


class OamTopkArgs(ctypes.Structure):
    _fields_ = [("kv", AttnKvGeom), ("G", i32), ("q", vp), ("k", vp), ("v", vp), ("kv_dtype", i32), ("k_scale", vp),
                ("k_part_tokens", i32), ("k_scale_stride", i32), ("v_scale", f32), ("vlog", vp), ("vlog_stride", i32),
                ("softmax_scale", f32), ("beta", f32), ("eps", f32), ("top_k", i32), ("block_tokens", i32),
                ("idx_out", vp),
                ("n_kept", vp), ("scores_out", vp), ("workspace", vp), ("workspace_bytes", sz)]


# Every entry point of the header, with its ctypes signature.
SIGNATURES = {
    "attn_decode_workspace_size": ([ctypes.POINTER(AttnDecodeArgs), ctypes.POINTER(sz)], i32),
    "attn_decode_split_tokens": ([ctypes.POINTER(AttnDecodeArgs), ctypes.POINTER(i32)], i32),
    "attn_decode_splitkv": ([ctypes.POINTER(AttnDecodeArgs), vp], i32),
    "attn_decode_splitkv_profiled": ([ctypes.POINTER(AttnDecodeArgs), vp, ctypes.POINTER(vp * 3)], i32),
    "attn_decode_splitkv_noalloc": ([ctypes.POINTER(AttnDecodeArgs), vp], i32),
    "attn_merge_lse": ([vp, vp, vp, vp, i32, i32, i32, vp, vp, vp], i32),
    "kv_quant_int8_workspace_size": ([ctypes.POINTER(AttnKvGeom), i32, ctypes.POINTER(sz)], i32),
    "kv_quant_int8": ([ctypes.POINTER(AttnKvGeom), vp, i32, i32, vp, vp, vp, sz, vp], i32),
    "oam_value_lognorm": ([ctypes.POINTER(AttnKvGeom), vp, i32, f32, f32, vp, i32, vp], i32),
    "oam_score_topk_workspace_size": ([ctypes.POINTER(OamTopkArgs), ctypes.POINTER(sz)], i32),
    "oam_score_topk": ([ctypes.POINTER(OamTopkArgs), vp], i32),
    "attn_status_string": ([i32], ctypes.c_char_p),
    "attn_last_error": ([], ctypes.c_char_p),
    "attn_util_copy": ([vp, vp, sz, vp], i32),
    "attn_util_read": ([vp, sz, vp, vp], i32),
}

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {detail or 'error'} (status {status})")
        self.status = status


def load(path: str = LIB_PATH):
    """Load the HIP library; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with long_context_decode_gqa_amd.build.build() "
                          "(this package has no CPU or eager fallback)")
    L = ctypes.CDLL(path)
    for name, (argtypes, restype) in SIGNATURES.items():
        fn = getattr(L, name)
        fn.argtypes = argtypes
        fn.restype = restype
    _lib = L
    return L


def check(status: int, where: str):
    if status != ATTN_OK:
        L = load()
        raise AttnError(status, where, L.attn_last_error().decode())
