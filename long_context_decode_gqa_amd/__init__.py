"""Single-query GQA decode attention for MI355X (gfx950).

Thin Python binding over the C ABI of ``libattn_decode.so`` (see
``include/attn_decode.h``): it only marshals torch device tensors into the ABI
structs and calls the library on the current HIP stream.  Every step of the
computation runs in the library's HIP kernels; if the library is missing the
import of the binding's entry points raises (there is no CPU fallback).
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib
from ._lib import ATTN_BF16, ATTN_F32, ATTN_I8, AttnError  # noqa: F401
from ._lib import ATTN_QUANT_EXACT as QUANT_EXACT, ATTN_QUANT_ROW as QUANT_ROW  # noqa: F401
from ._lib import ATTN_QUANT_STATIC as QUANT_STATIC  # noqa: F401

NOALLOC_SCRATCH_BYTES = 64 << 20  # attn_decode_splitkv_noalloc's static scratch per GPU

__all__ = ["KVGeometry", "attn_decode_splitkv", "attn_decode_splitkv_noalloc", "attn_merge_lse", "kv_quant_int8", "oam_value_lognorm",
           "oam_score_topk", "decode_workspace_size", "oam_workspace_size", "prepare_decode", "util_copy",
           "util_read", "decode_split_tokens", "AttnError"]

_DT = {torch.float32: ATTN_F32, torch.bfloat16: ATTN_BF16, torch.int8: ATTN_I8}


def _code(t: torch.Tensor) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported tensor dtype {t.dtype}") from None


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


@dataclass
class KVGeometry:
    """KV-cache geometry: row (b, kh, t) starts at element seq_offset[b] + kh*stride_h + t*stride_t.

    ``seq_lens`` (int32) and ``seq_offset`` (int64) are device tensors of length B.  A paged cache
    gives ``block_table`` (device int32 [B, table_stride]) instead of ``seq_offset``: row (b, kh, t)
    then starts at block_table[b, t // page_tokens] * page_stride + kh*stride_h
    + (t % page_tokens)*stride_t.
    """
    B: int
    KH: int
    D: int
    max_seq_len: int
    seq_lens: torch.Tensor
    seq_offset: Optional[torch.Tensor]
    stride_h: int
    stride_t: int
    block_table: Optional[torch.Tensor] = None
    page_tokens: int = 0
    page_stride: int = 0

    def c(self) -> _lib.AttnKvGeom:
        if self.B:
            assert self.seq_lens.dtype == torch.int32
            assert self.seq_offset is None or self.seq_offset.dtype == torch.int64
        g = _lib.AttnKvGeom(self.B, self.KH, self.D, self.max_seq_len, _ptr(self.seq_lens), _ptr(self.seq_offset),
                            self.stride_h, self.stride_t)
        if self.block_table is not None:
            assert self.block_table.dtype == torch.int32 and self.block_table.dim() == 2
            g.block_table = _ptr(self.block_table)
            g.page_tokens = self.page_tokens
            g.table_stride = self.block_table.shape[1]
            g.page_stride = self.page_stride
        return g

    @staticmethod
    def dense(B: int, KH: int, L: int, D: int, device="cuda") -> "KVGeometry":
        """[B][KH][L][D] caches, every sequence of length L."""
        lens = torch.full((B,), L, dtype=torch.int32, device=device)
        so = torch.arange(B, dtype=torch.int64, device=device) * (KH * L * D)
        return KVGeometry(B, KH, D, L, lens, so, L * D, D)


def _decode_args(q, k, v, geom: KVGeometry, G, out, lse, k_scale, k_part_tokens, k_scale_stride, v_scale,
                 token_idx, n_idx, idx_stride, softmax_scale, split_tokens, workspace, q_quant=0, q_scale=0.0,
                 q_rows=1, fixed_splits=0):
    a = _lib.AttnDecodeArgs()
    a.kv = geom.c()
    a.G = G
    a.q_rows = q_rows
    a.q_dtype, a.kv_dtype, a.out_dtype = _code(q), _code(k), _code(out)
    a.q, a.k, a.v = _ptr(q), _ptr(k), _ptr(v)
    a.k_scale = _ptr(k_scale)
    a.k_part_tokens = k_part_tokens
    a.k_scale_stride = k_scale_stride
    a.v_scale = v_scale
    a.q_quant, a.q_scale = q_quant, q_scale
    a.token_idx, a.n_idx, a.idx_stride = _ptr(token_idx), _ptr(n_idx), idx_stride
    a.softmax_scale = softmax_scale
    a.split_tokens = split_tokens
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    a.out, a.lse = _ptr(out), _ptr(lse)
    a.fixed_splits = fixed_splits
    return a


def decode_workspace_size(args: _lib.AttnDecodeArgs) -> int:
    n = ctypes.c_size_t(0)
    _lib.check(_lib.load().attn_decode_workspace_size(ctypes.byref(args), ctypes.byref(n)),
               "attn_decode_workspace_size")
    return n.value


def decode_split_tokens(args: _lib.AttnDecodeArgs) -> int:
    n = ctypes.c_int32(0)
    _lib.check(_lib.load().attn_decode_split_tokens(ctypes.byref(args), ctypes.byref(n)), "attn_decode_split_tokens")
    return n.value


class PreparedDecode:
    """A validated argument block; calling it enqueues one decode step on a stream."""

    def __init__(self, args: _lib.AttnDecodeArgs, keep, noalloc: bool = False):
        self.args = args
        self._keep = keep
        self._name = "attn_decode_splitkv_noalloc" if noalloc else "attn_decode_splitkv"
        self._fn = getattr(_lib.load(), self._name)

    def __call__(self, stream=None):
        _lib.check(self._fn(ctypes.byref(self.args), _stream(stream)), self._name)

    @property
    def split_tokens(self) -> int:
        """The chunk length the library uses for this call (its default when 0 was asked)."""
        return decode_split_tokens(self.args)

    def profiled(self, events, stream=None):
        """Same call, recording three torch.cuda.Event marks around the decode and merge launches."""
        arr = (ctypes.c_void_p * 3)(*[None if e is None else e.cuda_event for e in events])
        st = _lib.load().attn_decode_splitkv_profiled(ctypes.byref(self.args), _stream(stream), ctypes.byref(arr))
        _lib.check(st, "attn_decode_splitkv_profiled")


def prepare_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, geom: KVGeometry, G: int, *,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   out_dtype: torch.dtype = torch.float32, k_scale: Optional[torch.Tensor] = None,
                   k_part_tokens: int = 64, k_scale_stride: Optional[int] = None, v_scale: float = 1.0,
                   token_idx: Optional[torch.Tensor] = None, n_idx: Optional[torch.Tensor] = None,
                   idx_stride: Optional[int] = None, softmax_scale: float = 0.0, split_tokens: int = 0,
                   q_quant: int = 0, q_scale: float = 0.0, q_rows: int = 1, fixed_splits: int = 0,
                   workspace: Optional[torch.Tensor] = None, noalloc: bool = False) -> PreparedDecode:
    """Build (and allocate outputs/workspace for) one ``attn_decode_splitkv`` call.

    With int8 KV, ``k_part_tokens=0`` selects one per-tensor K scale (``k_scale[0]``) and
    ``q_quant`` (QUANT_EXACT / QUANT_ROW / QUANT_STATIC, with ``q_scale``) how the query is
    quantised.  ``q_rows`` > 1 is a multi-row (speculative) step: q, out and lse are
    [B, q_rows, KH*G, ...] and row r attends to the first L - (q_rows - 1) + r tokens.
    ``fixed_splits`` > 0 selects the unbalanced schedule (every (b, kh) in that many splits).
    ``noalloc`` calls ``attn_decode_splitkv_noalloc`` instead, which takes no workspace (the
    library's static scratch holds the partials); outputs not given are still allocated here."""
    dev = q.device
    QH = geom.KH * G
    if out is None:
        shape = (geom.B, QH, geom.D) if q_rows <= 1 else (geom.B, q_rows, QH, geom.D)
        out = torch.empty(shape, dtype=out_dtype, device=dev)
    if k_scale_stride is None:
        k_scale_stride = (max(1, -(-geom.max_seq_len // k_part_tokens))
                          if k_scale is not None and k_part_tokens > 0 else 0)
    if token_idx is not None and idx_stride is None:
        idx_stride = token_idx.shape[-1]
    a = _decode_args(q, k, v, geom, G, out, lse, k_scale, k_part_tokens, k_scale_stride, v_scale, token_idx, n_idx,
                     idx_stride or 0, softmax_scale, split_tokens, None, q_quant, q_scale, q_rows, fixed_splits)
    if noalloc:
        if workspace is not None:
            raise ValueError("noalloc takes no workspace")
    else:
        need = decode_workspace_size(a)
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = workspace.numel()
    p = PreparedDecode(a, [q, k, v, geom, out, lse, k_scale, token_idx, n_idx, workspace], noalloc)
    p.out, p.lse, p.workspace = out, lse, workspace
    return p


def attn_decode_splitkv(q, k, v, geom: KVGeometry, G: int, stream=None, **kw):
    """Split-KV decode attention; returns (out [B, KH*G, D], lse or None).  See prepare_decode for options."""
    p = prepare_decode(q, k, v, geom, G, **kw)
    p(stream)
    return p.out, p.lse


def attn_decode_splitkv_noalloc(q, k, v, geom: KVGeometry, G: int, stream=None, **kw):
    """attn_decode_splitkv through the entry point that takes no workspace (the library's static
    scratch, NOALLOC_SCRATCH_BYTES per GPU); pass ``out`` (and ``lse``) to allocate nothing here either."""
    p = prepare_decode(q, k, v, geom, G, noalloc=True, **kw)
    p(stream)
    return p.out, p.lse


def attn_merge_lse(o_part: torch.Tensor, m_part: torch.Tensor, l_part: torch.Tensor, row_split_start: torch.Tensor,
                   out_dtype: torch.dtype = torch.float32, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, stream=None):
    """Log-sum-exp merge of partial (m, l, o) triples laid out by a CSR row index."""
    rows = row_split_start.numel() - 1
    D = o_part.shape[-1]
    if out is None:
        out = torch.empty((rows, D), dtype=out_dtype, device=o_part.device)
    st = _lib.load().attn_merge_lse(_ptr(o_part), _ptr(m_part), _ptr(l_part), _ptr(row_split_start), rows, D,
                                    _code(out), _ptr(out), _ptr(lse), _stream(stream))
    _lib.check(st, "attn_merge_lse")
    return out, lse


def kv_quant_int8(x: torch.Tensor, geom: KVGeometry, partition_tokens: int = 64, codes=None, scales=None,
                  scale_stride: Optional[int] = None, workspace=None, stream=None):
    """INT8 codes (same geometry as x) and fp32 scales; partition_tokens = 0 gives one per-tensor scale."""
    L = _lib.load()
    if codes is None:
        codes = torch.zeros(x.shape, dtype=torch.int8, device=x.device)
    if partition_tokens > 0:
        if scale_stride is None:
            scale_stride = max(1, -(-geom.max_seq_len // partition_tokens))
        if scales is None:
            scales = torch.zeros(geom.B * geom.KH * scale_stride, dtype=torch.float32, device=x.device)
    else:
        scale_stride = 1
        if scales is None:
            scales = torch.zeros(1, dtype=torch.float32, device=x.device)
    g = geom.c()
    n = ctypes.c_size_t(0)
    _lib.check(L.kv_quant_int8_workspace_size(ctypes.byref(g), partition_tokens, ctypes.byref(n)),
               "kv_quant_int8_workspace_size")
    if n.value and workspace is None:
        workspace = torch.empty(max(256, n.value), dtype=torch.uint8, device=x.device)
    st = L.kv_quant_int8(ctypes.byref(g), _ptr(x), partition_tokens, scale_stride, _ptr(codes), _ptr(scales),
                         _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(stream))
    _lib.check(st, "kv_quant_int8")
    return codes, scales


def oam_value_lognorm(v: torch.Tensor, geom: KVGeometry, eps: float = 1e-6, vlog=None,
                      vlog_stride: Optional[int] = None, stream=None, v_scale: float = 1.0):
    """ln(||v_t|| + eps) per V row -> fp32 [B*KH, vlog_stride]; an int8 ``v`` holds codes of scale ``v_scale``."""
    if vlog_stride is None:
        vlog_stride = max(1, geom.max_seq_len)
    if vlog is None:
        vlog = torch.zeros((geom.B * geom.KH, vlog_stride), dtype=torch.float32, device=v.device)
    g = geom.c()
    st = _lib.load().oam_value_lognorm(ctypes.byref(g), _ptr(v), _code(v), v_scale, eps, _ptr(vlog), vlog_stride,
                                       _stream(stream))
    _lib.check(st, "oam_value_lognorm")
    return vlog


def _oam_args(q, k, geom, G, top_k, v, vlog, vlog_stride, softmax_scale, beta, eps, idx_out, n_kept, scores_out,
              workspace, k_scale=None, k_part_tokens=0, k_scale_stride=0, v_scale=1.0, block_tokens=0):
    a = _lib.OamTopkArgs()
    a.kv = geom.c()
    a.G = G
    a.q, a.k, a.v, a.vlog = _ptr(q), _ptr(k), _ptr(v), _ptr(vlog)
    a.kv_dtype = _code(k)
    a.k_scale, a.k_part_tokens, a.k_scale_stride, a.v_scale = _ptr(k_scale), k_part_tokens, k_scale_stride, v_scale
    a.vlog_stride = vlog_stride
    a.softmax_scale, a.beta, a.eps = softmax_scale, beta, eps
    a.top_k = top_k
    a.block_tokens = block_tokens
    a.idx_out, a.n_kept, a.scores_out = _ptr(idx_out), _ptr(n_kept), _ptr(scores_out)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel()
    return a


def oam_workspace_size(args: _lib.OamTopkArgs) -> int:
    n = ctypes.c_size_t(0)
    _lib.check(_lib.load().oam_score_topk_workspace_size(ctypes.byref(args), ctypes.byref(n)),
               "oam_score_topk_workspace_size")
    return n.value


class PreparedOam:
    def __init__(self, args, keep):
        self.args = args
        self._keep = keep
        self._fn = _lib.load().oam_score_topk

    def __call__(self, stream=None):
        _lib.check(self._fn(ctypes.byref(self.args), _stream(stream)), "oam_score_topk")


def prepare_oam(q, k, geom: KVGeometry, G: int, top_k: int, *, v=None, vlog=None, vlog_stride: Optional[int] = None,
                softmax_scale: float = 0.0, beta: float = 1.0, eps: float = 1e-6, idx_out=None, n_kept=None,
                scores_out=None, workspace=None, k_scale=None, k_part_tokens: int = 64,
                k_scale_stride: Optional[int] = None, v_scale: float = 1.0, block_tokens: int = 0) -> PreparedOam:
    """One ``oam_score_topk`` call.  An int8 ``k`` (and ``v``) is an INT8 cache with the K scales of
    ``prepare_decode`` (``k_part_tokens=0``: one per-tensor scale) and the V scale ``v_scale``.
    ``block_tokens`` > 1 keeps the ``top_k`` best blocks of that many tokens instead of tokens."""
    dev = q.device
    if k_scale_stride is None:
        k_scale_stride = (max(1, -(-geom.max_seq_len // k_part_tokens))
                          if k_scale is not None and k_part_tokens > 0 else 0)
    npairs = geom.B * geom.KH
    if idx_out is None:
        idx_out = torch.empty((npairs, top_k * max(block_tokens, 1)), dtype=torch.int32, device=dev)
    if n_kept is None:
        n_kept = torch.empty(npairs, dtype=torch.int32, device=dev)
    if vlog is not None and vlog_stride is None:
        vlog_stride = vlog.shape[-1]
    a = _oam_args(q, k, geom, G, top_k, v, vlog, vlog_stride or 0, softmax_scale, beta, eps, idx_out, n_kept,
                  scores_out, None, k_scale, k_part_tokens if k_scale is not None else 0, k_scale_stride, v_scale,
                  block_tokens)
    need = oam_workspace_size(a)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel()
    p = PreparedOam(a, [q, k, v, vlog, geom, idx_out, n_kept, scores_out, workspace, k_scale])
    p.idx_out, p.n_kept, p.scores_out, p.workspace = idx_out, n_kept, scores_out, workspace
    return p


def oam_score_topk(q, k, geom: KVGeometry, G: int, top_k: int, stream=None, **kw):
    """OAM scores and per-(b, kh) top-K kept indices; returns (idx_out [B*KH, top_k], n_kept [B*KH])."""
    p = prepare_oam(q, k, geom, G, top_k, **kw)
    p(stream)
    return p.idx_out, p.n_kept


def util_copy(dst: torch.Tensor, src: torch.Tensor, nbytes: Optional[int] = None, stream=None):
    n = src.numel() * src.element_size() if nbytes is None else nbytes
    _lib.check(_lib.load().attn_util_copy(_ptr(dst), _ptr(src), n, _stream(stream)), "attn_util_copy")


def util_read(src: torch.Tensor, sink: torch.Tensor, nbytes: Optional[int] = None, stream=None):
    n = src.numel() * src.element_size() if nbytes is None else nbytes
    _lib.check(_lib.load().attn_util_read(_ptr(src), n, _ptr(sink), _stream(stream)), "attn_util_read")
