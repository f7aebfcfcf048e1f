"""CPU oracle for single-query GQA decode attention — TEST INFRASTRUCTURE ONLY.

A ctypes front end to ``oracle.cpp`` (plain fp64 C++).  Only the tests, the
package smoke check and the benchmark's CPU-baseline leg may import this
module; the product library never calls it.  Inputs are numpy arrays that
the caller owns (bf16 is carried as uint16 bit patterns).
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
# ORACLE_LIB points the loader at another build of oracle.cpp (the sanitizer test builds one with
# AddressSanitizer and UndefinedBehaviorSanitizer and runs the pins against it)
_LIB = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

F32, BF16, I8 = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile liboracle.so with strict IEEE semantics (no contraction, no fast-math)."""
    if force or not os.path.exists(_LIB):
        cmd = ["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
               "-pthread", _SRC, "-o", _LIB + ".tmp"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


class _Problem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("KH", ctypes.c_int32), ("G", ctypes.c_int32), ("D", ctypes.c_int32),
        ("lens", ctypes.c_void_p), ("seq_offset", ctypes.c_void_p),
        ("stride_h", ctypes.c_int64), ("stride_t", ctypes.c_int64),
        ("q_type", ctypes.c_int32), ("kv_type", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p), ("k_part", ctypes.c_int32), ("k_scale_stride", ctypes.c_int32),
        ("v_scale", ctypes.c_float), ("softmax_scale", ctypes.c_double),
        ("tok_idx", ctypes.c_void_p), ("n_idx", ctypes.c_void_p), ("idx_stride", ctypes.c_int32),
        ("q_scale", ctypes.c_void_p),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        P = ctypes.POINTER(_Problem)
        vp, i32, i64, f64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.oracle_attention_rows.argtypes = [P, i32, vp, vp, vp, vp, i32]
        L.oracle_attention_rows_online.argtypes = [P, i32, vp, vp, i32, vp, vp]
        L.oracle_partial.argtypes = [P, i32, i32, i32, i32, vp, vp, vp]
        L.oracle_merge.argtypes = [i32, i32, vp, vp, vp, vp, vp]
        L.oracle_quant_partitions.argtypes = [i32, i32, i32, vp, vp, i64, i64, vp, i32, vp, vp, i32]
        L.oracle_quant_tensor.argtypes = [i32, i32, i32, vp, vp, i64, i64, vp, vp, vp]
        L.oracle_quant_rows.argtypes = [i32, i32, vp, vp, vp]
        L.oracle_quant_static.argtypes = [i64, vp, ctypes.c_float, vp]
        L.oracle_oam_scores.argtypes = [P, i32, i32, f64, f64, vp]
        L.oracle_value_lognorm.argtypes = [P, i32, i32, f64, vp]
        L.oracle_topk_sort.argtypes = [vp, i32, i32, vp]
        L.oracle_topk_sort.restype = i32
        L.oracle_topk_select.argtypes = [vp, i32, i32, vp]
        L.oracle_topk_select.restype = i32
        L.oracle_block_select.argtypes = [P, i32, i32, i32, i32, f64, f64, vp, vp]
        L.oracle_block_select.restype = i32
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.int8:
        return I8
    raise TypeError(f"unsupported element type {a.dtype}")


@dataclass
class Problem:
    """A decode problem held in host numpy arrays.

    K/V row (b, kh, t) starts at element seq_offset[b] + kh*stride_h + t*stride_t
    of the flat arrays ``k``/``v``.  ``q`` is [B, KH*G, D].  bf16 is uint16 bits.
    An int8 ``q`` holds codes; row (b, qh) is multiplied by q_scale[b*KH*G + qh].
    """
    B: int
    KH: int
    G: int
    D: int
    lens: np.ndarray
    seq_offset: np.ndarray
    stride_h: int
    stride_t: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    softmax_scale: float
    k_scale: Optional[np.ndarray] = None
    k_part: int = 64
    k_scale_stride: int = 1
    v_scale: float = 1.0
    tok_idx: Optional[np.ndarray] = None
    n_idx: Optional[np.ndarray] = None
    idx_stride: int = 0
    q_scale: Optional[np.ndarray] = None

    def _struct(self) -> _Problem:
        self._keep = [np.ascontiguousarray(self.lens, dtype=np.int32),
                      np.ascontiguousarray(self.seq_offset, dtype=np.int64)]
        s = _Problem()
        s.B, s.KH, s.G, s.D = self.B, self.KH, self.G, self.D
        s.lens, s.seq_offset = _ptr(self._keep[0]), _ptr(self._keep[1])
        s.stride_h, s.stride_t = self.stride_h, self.stride_t
        s.q_type, s.kv_type = _dtype_code(self.q), _dtype_code(self.k)
        if _dtype_code(self.v) != s.kv_type:
            raise TypeError("K and V must share an element type")
        for a in (self.q, self.k, self.v):
            if not a.flags["C_CONTIGUOUS"]:
                raise ValueError("arrays must be contiguous")
        s.q, s.k, s.v = _ptr(self.q), _ptr(self.k), _ptr(self.v)
        if self.k_scale is not None:
            ks = np.ascontiguousarray(self.k_scale, dtype=np.float32)
            self._keep.append(ks)
            s.k_scale = _ptr(ks)
        s.k_part, s.k_scale_stride, s.v_scale = self.k_part, self.k_scale_stride, self.v_scale
        s.softmax_scale = self.softmax_scale
        if self.tok_idx is not None:
            ti = np.ascontiguousarray(self.tok_idx, dtype=np.int32)
            ni = np.ascontiguousarray(self.n_idx, dtype=np.int32)
            self._keep += [ti, ni]
            s.tok_idx, s.n_idx, s.idx_stride = _ptr(ti), _ptr(ni), self.idx_stride
        if self.q_scale is not None:
            qs = np.ascontiguousarray(self.q_scale, dtype=np.float32)
            self._keep.append(qs)
            s.q_scale = _ptr(qs)
        return s


def attention_rows(p: Problem, rows: Sequence[tuple], nthreads: int = 1):
    """Plain-definition decode attention of the listed (b, qh) rows -> (out [n, D], lse [n])."""
    rb = np.array([r[0] for r in rows], dtype=np.int32)
    rq = np.array([r[1] for r in rows], dtype=np.int32)
    out = np.zeros((len(rows), p.D), dtype=np.float64)
    lse = np.zeros(len(rows), dtype=np.float64)
    s = p._struct()
    rc = lib().oracle_attention_rows(ctypes.byref(s), len(rows), _ptr(rb), _ptr(rq), _ptr(out), _ptr(lse),
                                     int(nthreads))
    if rc:
        raise ValueError("oracle_attention_rows: invalid arguments")
    return out, lse


def attention_multirow(p: Problem, q_rows: int, rows: Sequence[tuple], nthreads: int = 1):
    """Multi-row (speculative) decode, the NV blog's (1 + draft) x G GEMM-M: ``p.q`` is
    [B, R, KH*G, D] (int8 ``q_scale`` then [B, R, KH*G]); the R query tokens are the last R tokens
    of each cache, so row (b, r, qh) attends to the first L_b - (R - 1) + r tokens (itself and
    what precedes it).  Each row is the plain definition on that prefix.  rows: (b, r, qh)."""
    R = int(q_rows)
    out = np.zeros((len(rows), p.D), dtype=np.float64)
    lse = np.zeros(len(rows), dtype=np.float64)
    q = np.asarray(p.q).reshape(p.B, R, p.KH * p.G, p.D)
    for r in range(R):
        sel = [i for i, row in enumerate(rows) if row[1] == r]
        if not sel:
            continue
        lens_r = np.maximum(np.asarray(p.lens, np.int64) - (R - 1) + r, 0).astype(np.int32)
        qs = None if p.q_scale is None else np.ascontiguousarray(
            np.asarray(p.q_scale).reshape(p.B, R, p.KH * p.G)[:, r]).reshape(-1)
        pr = dataclasses.replace(p, q=np.ascontiguousarray(q[:, r]), lens=lens_r, q_scale=qs)
        o, l = attention_rows(pr, [(rows[i][0], rows[i][2]) for i in sel], nthreads)
        out[sel] = o
        lse[sel] = l
    return out, lse


def all_rows(p: Problem):
    return [(b, qh) for b in range(p.B) for qh in range(p.KH * p.G)]


def attention_rows_online(p: Problem, rows: Sequence[tuple], block: int):
    rb = np.array([r[0] for r in rows], dtype=np.int32)
    rq = np.array([r[1] for r in rows], dtype=np.int32)
    out = np.zeros((len(rows), p.D), dtype=np.float64)
    lse = np.zeros(len(rows), dtype=np.float64)
    s = p._struct()
    if lib().oracle_attention_rows_online(ctypes.byref(s), len(rows), _ptr(rb), _ptr(rq), int(block),
                                          _ptr(out), _ptr(lse)):
        raise ValueError("oracle_attention_rows_online: invalid arguments")
    return out, lse


def partial(p: Problem, b: int, qh: int, t0: int, t1: int):
    m = np.zeros(1)
    l = np.zeros(1)
    o = np.zeros(p.D)
    s = p._struct()
    if lib().oracle_partial(ctypes.byref(s), b, qh, t0, t1, _ptr(m), _ptr(l), _ptr(o)):
        raise ValueError("oracle_partial: invalid arguments")
    return float(m[0]), float(l[0]), o


def merge(m: np.ndarray, l: np.ndarray, o: np.ndarray):
    m = np.ascontiguousarray(m, dtype=np.float64)
    l = np.ascontiguousarray(l, dtype=np.float64)
    o = np.ascontiguousarray(o, dtype=np.float64)
    n, D = o.shape
    out = np.zeros(D)
    lse = np.zeros(1)
    if lib().oracle_merge(n, D, _ptr(m), _ptr(l), _ptr(o), _ptr(out), _ptr(lse)):
        raise ValueError("oracle_merge: invalid arguments")
    return out, float(lse[0])


def quant_partitions(B, KH, D, lens, seq_offset, stride_h, stride_t, x_bf16: np.ndarray, part: int,
                     scale_stride: int):
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    so = np.ascontiguousarray(seq_offset, dtype=np.int64)
    codes = np.zeros(x_bf16.shape, dtype=np.int8)
    scales = np.zeros(B * KH * scale_stride, dtype=np.float32)
    if lib().oracle_quant_partitions(B, KH, D, _ptr(lens), _ptr(so), stride_h, stride_t, _ptr(x_bf16), part,
                                     _ptr(codes), _ptr(scales), scale_stride):
        raise ValueError("oracle_quant_partitions: invalid arguments")
    return codes, scales


def quant_rows(x_bf16: np.ndarray):
    """Per-row INT8 of a [rows, D] bf16 array (the query of Schemes A and B) -> (codes, scales)."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, D = x.shape
    codes = np.zeros(x.shape, dtype=np.int8)
    scales = np.zeros(rows, dtype=np.float32)
    if lib().oracle_quant_rows(rows, D, _ptr(x), _ptr(codes), _ptr(scales)):
        raise ValueError("oracle_quant_rows: invalid arguments")
    return codes, scales


def quant_static(x_bf16: np.ndarray, scale: float) -> np.ndarray:
    """INT8 codes of bf16 values with a given per-tensor scale (the baseline scheme)."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    codes = np.zeros(x.shape, dtype=np.int8)
    if lib().oracle_quant_static(x.size, _ptr(x), float(scale), _ptr(codes)):
        raise ValueError("oracle_quant_static: invalid arguments")
    return codes


def quant_tensor(B, KH, D, lens, seq_offset, stride_h, stride_t, x_bf16: np.ndarray):
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    so = np.ascontiguousarray(seq_offset, dtype=np.int64)
    codes = np.zeros(x_bf16.shape, dtype=np.int8)
    scale = np.zeros(1, dtype=np.float32)
    if lib().oracle_quant_tensor(B, KH, D, _ptr(lens), _ptr(so), stride_h, stride_t, _ptr(x_bf16),
                                 _ptr(codes), _ptr(scale)):
        raise ValueError("oracle_quant_tensor: invalid arguments")
    return codes, float(scale[0])


def oam_scores(p: Problem, b: int, kh: int, beta: float, eps: float) -> np.ndarray:
    out = np.zeros(int(p.lens[b]), dtype=np.float64)
    s = p._struct()
    if lib().oracle_oam_scores(ctypes.byref(s), b, kh, float(beta), float(eps), _ptr(out)):
        raise ValueError("oracle_oam_scores: invalid arguments")
    return out


def value_lognorm(p: Problem, b: int, kh: int, eps: float) -> np.ndarray:
    out = np.zeros(int(p.lens[b]), dtype=np.float64)
    s = p._struct()
    if lib().oracle_value_lognorm(ctypes.byref(s), b, kh, float(eps), _ptr(out)):
        raise ValueError("oracle_value_lognorm: invalid arguments")
    return out


def topk_sort(scores: np.ndarray, k: int) -> np.ndarray:
    scores = np.ascontiguousarray(scores, dtype=np.float64)
    idx = np.zeros(max(1, min(k, len(scores))), dtype=np.int32)
    n = lib().oracle_topk_sort(_ptr(scores), len(scores), int(k), _ptr(idx))
    if n < 0:
        raise ValueError("oracle_topk_sort: invalid arguments")
    return idx[:n].copy()


def topk_select(scores: np.ndarray, k: int) -> np.ndarray:
    scores = np.ascontiguousarray(scores, dtype=np.float64)
    idx = np.zeros(max(1, min(k, len(scores))), dtype=np.int32)
    n = lib().oracle_topk_select(_ptr(scores), len(scores), int(k), _ptr(idx))
    if n < 0:
        raise ValueError("oracle_topk_select: invalid arguments")
    return idx[:n].copy()


def block_select(p: Problem, b: int, kh: int, block_tokens: int, n_blocks: int, beta: float = 0.0,
                 eps: float = 1e-6):
    """Block-granular top-n selection -> (kept token indices ascending, block scores)."""
    L = int(p.lens[b])
    idx = np.zeros(max(1, L), dtype=np.int32)
    bs = np.zeros(max(1, -(-L // block_tokens)), dtype=np.float64)
    s = p._struct()
    n = lib().oracle_block_select(ctypes.byref(s), b, kh, block_tokens, n_blocks, float(beta), float(eps),
                                  _ptr(idx), _ptr(bs))
    if n < 0:
        raise ValueError("oracle_block_select: invalid arguments")
    return idx[:n].copy(), bs[:-(-L // block_tokens)].copy()
