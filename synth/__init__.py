"""Seeded synthetic inputs for long-context GQA decode attention.

Draws random numbers and lays them out; holds none of the attention,
quantisation or token-selection arithmetic.  Shared by the oracle's tests and
the GPU tests/bench (the only code both sides use).  The generator itself is
``synth.c`` (splitmix64 counters + Box-Muller, see its header).

Workloads (the shapes the pages discuss: 32K/128K KV decode, GQA G=8 with
head size 128, 128K-next-to-512 ragged batches, INT8 KV with outlier
channels, output-aware token dropping at 128K):

=========  ==========================================================================
tiny       B=1, KH=1, G=4, D=64, L=1024, fp32 N(0,1); 4 splits of 256
gqa32k     B=16, KH=8, G=8, D=128, L=32768, bf16 N(0,1); 1024-token splits
ragged     32 sequences, L_b log-uniform in [512, 131072], KH=8, G=8, D=128, bf16,
           head-major packed cache
int8_128k  B=4, KH=8, G=8, D=128, L=131072; bf16 N(0,1) K/V with 2 outlier
           channels x10 per (tensor, KV head); K quantised per 64 tokens, V per tensor
oam_128k   B=4, KH=8, G=8, D=128, L=131072; K N(0,1); V = unit N(0,1) direction
           x exp(N(0,1)); beta=1, eps=1e-6, keep 4096
dense128k  B=4, KH=8, G=8, D=128, L=131072, bf16 N(0,1)
=========  ==========================================================================

split_tokens 0 means the library default (about one chunk per decode worker:
2048 tokens for the 128K, INT8 and ragged workloads).  gqa32k keeps the
1024-token split-KV chunks its definition names; the attention over OAM's
4096 kept tokens uses 128-token chunks.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")

# Stream ids ("tensor" argument of the counter generator).
T_Q, T_K, T_V, T_LENS, T_OUTLIERS, T_NORMS = 0, 1, 2, 3, 4, 5
NORMAL, UNIT_DIR_LOGNORMAL = 0, 1
F32, BF16 = 0, 1


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", _SRC, "-o", _LIB + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        u64, u32, i32, i64, vp = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        L.synth_uniform.argtypes = [u64, u32, u64]
        L.synth_uniform.restype = ctypes.c_double
        L.synth_normal.argtypes = [u64, u32, u64]
        L.synth_normal.restype = ctypes.c_double
        L.synth_word.argtypes = [u64, u32, u64]
        L.synth_word.restype = u64
        L.synth_fill.argtypes = [u64, u32, u32, i32, i32, i32, vp, vp, i64, i64, i32, vp, i32, vp, i32]
        L.synth_fill.restype = ctypes.c_int
        _lib = L
    return _lib


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def uniform(seed: int, tensor: int, i: int) -> float:
    return lib().synth_uniform(seed, tensor, i)


def normal(seed: int, tensor: int, i: int) -> float:
    return lib().synth_normal(seed, tensor, i)


def word(seed: int, tensor: int, i: int) -> int:
    return lib().synth_word(seed, tensor, i)


@dataclass
class Geometry:
    """Where K/V row (b, kh, t) lives: seq_offset[b] + kh*stride_h + t*stride_t (elements)."""
    B: int
    KH: int
    D: int
    lens: np.ndarray
    seq_offset: np.ndarray
    stride_h: int
    stride_t: int
    numel: int

    @property
    def max_len(self) -> int:
        return int(self.lens.max()) if self.B else 0


def dense_geometry(B: int, KH: int, L: int, D: int) -> Geometry:
    """[B][KH][L][D] layout."""
    lens = np.full(B, L, dtype=np.int32)
    so = np.arange(B, dtype=np.int64) * KH * L * D
    return Geometry(B, KH, D, lens, so, L * D, D, B * KH * L * D)


def packed_token_major_geometry(lens: np.ndarray, KH: int, D: int) -> Geometry:
    """Sequences packed one after another, token-major: [sum L][KH][D]."""
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    cum = np.concatenate([[0], np.cumsum(lens.astype(np.int64))])
    so = cum[:-1] * KH * D
    return Geometry(len(lens), KH, D, lens, so.astype(np.int64), D, KH * D, int(cum[-1]) * KH * D)


def packed_head_major_geometry(lens: np.ndarray, KH: int, D: int) -> Geometry:
    """[KH][sum L][D]: every head holds all sequences back to back."""
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    cum = np.concatenate([[0], np.cumsum(lens.astype(np.int64))])
    total = int(cum[-1])
    so = cum[:-1] * D
    return Geometry(len(lens), KH, D, lens, so.astype(np.int64), total * D, D, KH * total * D)


def fill(seed: int, tensor: int, geom: Geometry, fmt: int = BF16, kind: int = NORMAL,
         chan_mult: Optional[np.ndarray] = None, norm_tensor: int = T_NORMS,
         out: Optional[np.ndarray] = None, nthreads: Optional[int] = None) -> np.ndarray:
    """Fill a flat array of geom.numel elements (uint16 bf16 bits or float32)."""
    dt = np.uint16 if fmt == BF16 else np.float32
    if out is None:
        out = np.zeros(geom.numel, dtype=dt)
    assert out.dtype == dt and out.size >= geom.numel and out.flags["C_CONTIGUOUS"]
    lens = np.ascontiguousarray(geom.lens, dtype=np.int32)
    so = np.ascontiguousarray(geom.seq_offset, dtype=np.int64)
    cm = None
    if chan_mult is not None:
        cm = np.ascontiguousarray(chan_mult, dtype=np.float32)
        assert cm.shape == (geom.KH, geom.D)
    rc = lib().synth_fill(seed, tensor, norm_tensor, geom.B, geom.KH, geom.D,
                          lens.ctypes.data_as(ctypes.c_void_p), so.ctypes.data_as(ctypes.c_void_p),
                          geom.stride_h, geom.stride_t, kind,
                          None if cm is None else cm.ctypes.data_as(ctypes.c_void_p), fmt,
                          out.ctypes.data_as(ctypes.c_void_p), nthreads or default_threads())
    if rc:
        raise ValueError("synth_fill: invalid arguments")
    return out


def fill_q(seed: int, B: int, QH: int, D: int, fmt: int = BF16) -> np.ndarray:
    """Q [B, QH, D]: element (b, qh, d) is normal number ((b*QH + qh) << 40) + d of stream T_Q."""
    g = Geometry(B, QH, D, np.ones(B, np.int32), np.arange(B, dtype=np.int64) * QH * D, D, D, B * QH * D)
    return fill(seed, T_Q, g, fmt=fmt).reshape(B, QH, D)


def loguniform_lengths(seed: int, n: int, lo: int = 512, hi: int = 131072) -> np.ndarray:
    """L_b = floor(exp(ln lo + u_b ln(hi/lo))), u_b uniform from stream T_LENS, clamped to [lo, hi]."""
    out = np.zeros(n, dtype=np.int32)
    for b in range(n):
        u = uniform(seed, T_LENS, b)
        L = int(math.floor(math.exp(math.log(lo) + u * math.log(hi / lo))))
        out[b] = min(hi, max(lo, L))
    return out


def outlier_channels(seed: int, which: int, KH: int, D: int, count: int = 2):
    """`count` distinct channels per KV head for tensor `which` (0 = K, 1 = V)."""
    chans = []
    for kh in range(KH):
        picked = []
        i = (which * KH + kh) * 1024
        while len(picked) < count:
            c = int(word(seed, T_OUTLIERS, i) % D)
            i += 1
            if c not in picked:
                picked.append(c)
        chans.append(picked)
    return chans


def outlier_multipliers(seed: int, which: int, KH: int, D: int, count: int = 2, factor: float = 10.0):
    m = np.ones((KH, D), dtype=np.float32)
    for kh, cs in enumerate(outlier_channels(seed, which, KH, D, count)):
        for c in cs:
            m[kh, c] = factor
    return m


@dataclass
class Workload:
    name: str
    B: int
    KH: int
    G: int
    D: int
    seed: int
    dtype: str                 # "f32" or "bf16" element type of Q/K/V as generated
    lens: np.ndarray
    split_tokens: int = 1024   # 0: the library default
    layout: str = "dense"      # dense | token_major | head_major
    outliers: int = 0
    v_kind: int = NORMAL
    top_k: int = 0
    beta: float = 1.0
    eps: float = 1e-6
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def QH(self) -> int:
        return self.KH * self.G

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def geometry(self) -> Geometry:
        if self.layout == "dense":
            assert np.all(self.lens == self.lens[0])
            return dense_geometry(self.B, self.KH, int(self.lens[0]), self.D)
        if self.layout == "token_major":
            return packed_token_major_geometry(self.lens, self.KH, self.D)
        return packed_head_major_geometry(self.lens, self.KH, self.D)

    def kv_tokens(self) -> int:
        return int(np.sum(self.lens.astype(np.int64)))


def workload(name: str, **over) -> Workload:
    """The named synthetic workloads; keyword overrides give smaller variants."""
    if name == "tiny":
        w = Workload("tiny", 1, 1, 4, 64, 1, "f32", np.array([1024], np.int32), split_tokens=256)
    elif name == "gqa32k":
        w = Workload("gqa32k", 16, 8, 8, 128, 2, "bf16", np.full(16, 32768, np.int32), split_tokens=1024)
    elif name == "ragged":
        w = Workload("ragged", 32, 8, 8, 128, 3, "bf16", loguniform_lengths(3, 32), layout="head_major", split_tokens=0)
    elif name == "int8_128k":
        w = Workload("int8_128k", 4, 8, 8, 128, 4, "bf16", np.full(4, 131072, np.int32), outliers=2, split_tokens=0)
    elif name == "oam_128k":
        w = Workload("oam_128k", 4, 8, 8, 128, 5, "bf16", np.full(4, 131072, np.int32),
                     v_kind=UNIT_DIR_LOGNORMAL, top_k=4096, split_tokens=0)
    elif name == "dense128k":
        w = Workload("dense128k", 4, 8, 8, 128, 6, "bf16", np.full(4, 131072, np.int32), split_tokens=0)
    else:
        raise KeyError(name)
    for k, v in over.items():
        if k == "L":
            w.lens = np.full(w.B, int(v), np.int32)
        elif k == "B" and "L" not in over and "lens" not in over:
            w.B = int(v)
            w.lens = np.resize(w.lens, w.B).astype(np.int32)
        else:
            setattr(w, k, v)
    w.lens = np.ascontiguousarray(w.lens, dtype=np.int32)
    assert len(w.lens) == w.B
    return w


def generate(w: Workload, nthreads: Optional[int] = None):
    """Host arrays (q [B,QH,D], k flat, v flat, geometry) for a workload."""
    fmt = F32 if w.dtype == "f32" else BF16
    geom = w.geometry()
    q = fill_q(w.seed, w.B, w.QH, w.D, fmt)
    km = vm = None
    if w.outliers:
        km = outlier_multipliers(w.seed, 0, w.KH, w.D, w.outliers)
        vm = outlier_multipliers(w.seed, 1, w.KH, w.D, w.outliers)
    k = fill(w.seed, T_K, geom, fmt=fmt, chan_mult=km, nthreads=nthreads)
    v = fill(w.seed, T_V, geom, fmt=fmt, kind=w.v_kind, chan_mult=vm, nthreads=nthreads)
    return q, k, v, geom


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    return (a.astype(np.uint32) << 16).view(np.float32)
