"""Small builders shared by the tests (no attention arithmetic here)."""
import math

import numpy as np

import oracle
import synth


def dense_problem(q, k, v, softmax_scale=None, lens=None):
    """q [B, KH*G, D]; k, v [B, KH, L, D] (float32, uint16 bf16 bits or int8)."""
    B, KH, L, D = k.shape
    G = q.shape[1] // KH
    geom = synth.dense_geometry(B, KH, L, D)
    if lens is None:
        lens = geom.lens
    return oracle.Problem(B, KH, G, D, np.asarray(lens, np.int32), geom.seq_offset, geom.stride_h, geom.stride_t,
                          np.ascontiguousarray(q), np.ascontiguousarray(k).reshape(-1),
                          np.ascontiguousarray(v).reshape(-1),
                          1.0 / math.sqrt(D) if softmax_scale is None else softmax_scale)


def random_dense(seed, B, KH, G, D, L, fmt=synth.F32):
    geom = synth.dense_geometry(B, KH, L, D)
    q = synth.fill_q(seed, B, KH * G, D, fmt)
    k = synth.fill(seed, synth.T_K, geom, fmt=fmt).reshape(B, KH, L, D)
    v = synth.fill(seed, synth.T_V, geom, fmt=fmt).reshape(B, KH, L, D)
    return q, k, v


def with_tokens(p: oracle.Problem, idx_lists, stride=None):
    """Copy of p restricted to per-(b, kh) token lists (list over b*KH + kh)."""
    n = np.array([len(x) for x in idx_lists], dtype=np.int32)
    stride = stride or max(1, int(n.max()) if len(n) else 1)
    arr = np.zeros((len(idx_lists), stride), dtype=np.int32)
    for i, x in enumerate(idx_lists):
        arr[i, :len(x)] = x
    return oracle.Problem(p.B, p.KH, p.G, p.D, p.lens, p.seq_offset, p.stride_h, p.stride_t, p.q, p.k, p.v,
                          p.softmax_scale, p.k_scale, p.k_part, p.k_scale_stride, p.v_scale,
                          arr.reshape(-1), n, stride)
