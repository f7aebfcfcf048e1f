"""attn_decode_splitkv_noalloc, the decode entry point that takes no workspace (its partials
and counters live in the library's static scratch), against attn_decode_splitkv on the same
inputs.

GPU: calls in a row whose inputs shrink, so each call starts from the scratch contents the
previous one left: out and lse bit-equal to attn_decode_splitkv's (same kernels, same split),
and the smallest call also against the oracle.  CPU: the argument checks that run before any
device work (a workspace given, a call needing more scratch than the array holds, B = 0).
"""
import ctypes
import math

import numpy as np
import pytest
import torch

import long_context_decode_gqa_amd as pkg
import oracle
import synth
from long_context_decode_gqa_amd import _lib

FAKE = 0x10000  # never dereferenced: validation fails before any device work


def _host_args(B, L, **over):
    a = _lib.AttnDecodeArgs()
    a.kv = _lib.AttnKvGeom(B, 8, 128, L, FAKE, FAKE, max(L, 1) * 128, 128)
    a.G = 8
    a.q_dtype = a.kv_dtype = _lib.ATTN_BF16
    a.out_dtype = _lib.ATTN_F32
    a.q = a.k = a.v = a.out = FAKE
    for k, v in over.items():
        setattr(a, k, v)
    return a


def _noalloc_status(a):
    return _lib.load().attn_decode_splitkv_noalloc(ctypes.byref(a), None)


def test_noalloc_rejects_a_workspace_argument():
    a = _host_args(2, 4096, workspace=FAKE, workspace_bytes=1 << 20)
    assert _noalloc_status(a) == _lib.ATTN_ERR_INVALID_ARG
    assert b"workspace must be NULL" in _lib.load().attn_last_error()


def test_noalloc_rejects_calls_beyond_its_scratch():
    # 256 sequences x 8 KV heads x 131072 tokens need about 281 MB of partials
    a = _host_args(256, 131072)
    n = ctypes.c_size_t(0)
    assert _lib.load().attn_decode_workspace_size(ctypes.byref(a), ctypes.byref(n)) == 0
    assert n.value > pkg.NOALLOC_SCRATCH_BYTES
    assert _noalloc_status(a) == _lib.ATTN_ERR_WORKSPACE_TOO_SMALL
    msg = _lib.load().attn_last_error()
    assert str(n.value).encode() in msg and str(pkg.NOALLOC_SCRATCH_BYTES).encode() in msg


def test_noalloc_empty_batch_is_a_no_op():
    assert _noalloc_status(_host_args(0, 0)) == _lib.ATTN_OK


@pytest.mark.parametrize("over", [dict(G=0), dict(kv_dtype=7), dict(q_rows=-1), dict(split_tokens=48),
                                  dict(fixed_splits=-2), dict(out=0)])
def test_noalloc_argument_errors_match_the_workspace_entry_point(over):
    a = _host_args(2, 4096, **over)
    st = _noalloc_status(a)
    assert st != _lib.ATTN_OK
    a.workspace, a.workspace_bytes = FAKE, 1 << 30
    assert _lib.load().attn_decode_splitkv(ctypes.byref(a), None) == st


# --- GPU ---

DEV = torch.device("cuda:0")


def _to_dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _geom(g):
    return pkg.KVGeometry(g.B, g.KH, g.D, int(g.max_len) if g.B else 0, torch.from_numpy(g.lens).to(DEV),
                          torch.from_numpy(g.seq_offset).to(DEV), g.stride_h, g.stride_t)


def _both(name, w, q, k, v, g, **kw):
    """out and lse from both entry points; the no-allocation call's outputs start as NaN."""
    print(f"[case] noalloc {name}: B={w.B} KH={w.KH} G={w.G} D={w.D} max_len={int(g.max_len)} {kw}", flush=True)
    R = kw.get("q_rows", 1)
    qd = _to_dev(q.reshape(-1)).view(w.B, w.QH, w.D) if R == 1 else _to_dev(q.reshape(-1)).view(w.B, R, w.QH, w.D)
    geom = _geom(g)
    lse_shape = (w.B, w.QH) if R == 1 else (w.B, R, w.QH)
    lse_a = torch.empty(lse_shape, dtype=torch.float32, device=DEV)
    out_a, _ = pkg.attn_decode_splitkv(qd, k, v, geom, w.G, lse=lse_a, **kw)
    out_b = torch.full_like(out_a, float("nan"))
    lse_b = torch.full_like(lse_a, float("nan"))
    pkg.attn_decode_splitkv_noalloc(qd, k, v, geom, w.G, out=out_b, lse=lse_b, **kw)
    torch.cuda.synchronize()
    fmt = torch.int16 if out_a.dtype == torch.bfloat16 else torch.int32
    assert torch.equal(out_a.view(fmt), out_b.view(fmt)), "out differs from attn_decode_splitkv"
    assert torch.equal(lse_a.view(torch.int32), lse_b.view(torch.int32)), "lse differs from attn_decode_splitkv"
    return out_b, lse_b


@pytest.mark.gpu
def test_noalloc_matches_the_workspace_entry_point_on_shrinking_calls():
    # 1: the 32-sequence ragged batch (512 .. 131072 tokens, about 35 MB of partials)
    w = synth.workload("ragged")
    q, k, v, g = synth.generate(w)
    _both("ragged", w, q, _to_dev(k), _to_dev(v), g)
    del k, v
    # 2: smaller, other lengths (the scratch holds call 1's partials and counters)
    w = synth.workload("gqa32k", B=3, lens=np.array([9000, 130, 20000], np.int32), layout="head_major", seed=41)
    q, k, v, g = synth.generate(w)
    _both("three sequences", w, q, _to_dev(k), _to_dev(v), g, split_tokens=256)
    # 3: smaller still, bf16 output, one worker per sequence; checked against the oracle as well
    w = synth.workload("gqa32k", B=2, lens=np.array([700, 0], np.int32), G=4, D=64, layout="token_major", seed=42)
    q, k, v, g = synth.generate(w)
    out, lse = _both("two short sequences", w, q, _to_dev(k), _to_dev(v), g, out_dtype=torch.bfloat16)
    p = oracle.Problem(w.B, w.KH, w.G, w.D, g.lens, g.seq_offset, g.stride_h, g.stride_t, np.ascontiguousarray(q),
                       k, v, 1.0 / math.sqrt(w.D))
    ref, ref_lse = oracle.attention_rows(p, oracle.all_rows(p))
    o = out.float().cpu().numpy().reshape(-1, w.D)
    assert np.all(np.abs(o - ref) <= 2e-3 + np.abs(ref) * 2.0 ** -9)
    lh = lse.cpu().numpy().reshape(-1)
    fin = np.isfinite(ref_lse)
    assert np.all(np.isneginf(lh[~fin])) and np.abs(lh[fin] - ref_lse[fin]).max() <= 1e-3


@pytest.mark.gpu
def test_noalloc_int8_and_multirow_after_larger_calls():
    # INT8 cache (64-token K partitions, per-tensor V): larger first, then smaller
    for B, L, seed in ((4, 40000, 43), (2, 3000, 44)):
        w = synth.workload("int8_128k", B=B, L=L, seed=seed)
        q, k, v, g = synth.generate(w)
        geom = _geom(g)
        kc, ks = pkg.kv_quant_int8(_to_dev(k), geom, 64)
        vc, vs = pkg.kv_quant_int8(_to_dev(v), geom, 0)
        _both(f"int8 B={B} L={L}", w, q, kc, vc, g, k_scale=ks, k_part_tokens=64, v_scale=float(vs[0]))
    # multi-row (R = 4 query rows per sequence)
    w = synth.workload("gqa32k", B=2, lens=np.array([5000, 64], np.int32), layout="head_major", seed=45)
    _, k, v, g = synth.generate(w)
    q = synth.fill_q(46, w.B, 4 * w.QH, w.D, synth.BF16)
    _both("multirow R=4", w, q, _to_dev(k), _to_dev(v), g, q_rows=4)
