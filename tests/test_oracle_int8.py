"""Pins of the oracle's INT8 KV quantisation.

Source: "优化稀疏注意力中的令牌丢弃机制" §6: per-tensor q_val = round(val/scale),
val ~ q_val*scale; Scheme A's per-token-partition scale[i] = max|k[i*chunk:(i+1)*chunk]|/127
with 64- or 128-token partitions; V keeps one per-tensor scale.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth
from helpers import dense_problem, random_dense

to32 = synth.bf16_bits_to_f32


def _bf16(x):
    a = np.asarray(x, np.float32)
    u = a.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "golden values must be exact bf16"
    return (u >> 16).astype(np.uint16)


def test_hand_worked_codes_and_scales(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "int8_hand_examples.json")))
    toks = np.array(g["tokens"], np.float32)
    L, D, part = toks.shape[0], g["D"], g["part"]
    geom = synth.dense_geometry(1, 1, L, D)
    x = _bf16(toks).reshape(-1)
    codes, scales = oracle.quant_partitions(1, 1, D, geom.lens, geom.seq_offset, geom.stride_h, geom.stride_t,
                                            x, part, 3)
    np.testing.assert_array_equal(codes.reshape(L, D), np.array(g["codes"], np.int8))
    np.testing.assert_array_equal(scales, np.array(g["scales"], np.float32))


def _partition_case(seed=31, B=2, KH=2, D=16, lens=(130, 64), part=64, outlier=True):
    lens = np.array(lens, np.int32)
    geom = synth.packed_head_major_geometry(lens, KH, D)
    mult = synth.outlier_multipliers(seed, 0, KH, D) if outlier else None
    x = synth.fill(seed, synth.T_K, geom, chan_mult=mult)
    stride = max(1, -(-int(lens.max()) // part))
    codes, scales = oracle.quant_partitions(B, KH, D, geom.lens, geom.seq_offset, geom.stride_h, geom.stride_t,
                                            x, part, stride)
    return geom, x, codes, scales, stride


def _rows(geom, b, kh, t0, t1):
    base = geom.seq_offset[b] + kh * geom.stride_h
    return [base + t * geom.stride_t + np.arange(geom.D) for t in range(t0, t1)]


@pytest.mark.parametrize("part", [64, 128, 7])
def test_partition_max_maps_to_127_and_error_bound(part):
    geom, x, codes, scales, stride = _partition_case(part=part)
    xf = to32(x)
    for b in range(geom.B):
        for kh in range(geom.KH):
            for t0 in range(0, int(geom.lens[b]), part):
                t1 = min(int(geom.lens[b]), t0 + part)
                idx = np.concatenate(_rows(geom, b, kh, t0, t1))
                s = scales[(b * geom.KH + kh) * stride + t0 // part]
                vals, cs = xf[idx], codes[idx].astype(np.int32)
                amax = np.abs(vals).max()
                assert s == np.float32(amax) / np.float32(127)
                # the largest magnitude is exactly +-127 (fl32(A / fl32(A/127)) = 127)
                assert np.all(np.abs(cs[np.abs(vals) == amax]) == 127)
                assert np.all(np.abs(cs) <= 127)
                # reconstruction within half a step plus the fp32 quotient rounding
                err = np.abs(vals.astype(np.float64) - cs * np.float64(s))
                assert np.all(err <= np.float64(s) * (0.5 + 2.0 ** -17))


def test_partitions_align_at_token_zero_of_each_sequence():
    # Zeroing everything but one partition changes only that partition's scale.
    geom, x, codes, scales, stride = _partition_case(lens=(130, 64), part=64)
    x2 = x.copy()
    keep = np.concatenate(_rows(geom, 0, 1, 64, 128))
    mask = np.ones(x2.size, bool)
    mask[keep] = False
    x2[mask] = 0
    codes2, scales2 = oracle.quant_partitions(geom.B, geom.KH, geom.D, geom.lens, geom.seq_offset, geom.stride_h,
                                              geom.stride_t, x2, 64, stride)
    nz = np.nonzero(scales2)[0]
    assert list(nz) == [(0 * geom.KH + 1) * stride + 1]
    assert scales2[nz[0]] == scales[nz[0]]
    np.testing.assert_array_equal(codes2[keep], codes[keep])


def test_per_tensor_equals_one_partition_covering_everything():
    lens = np.array([200], np.int32)
    geom = synth.dense_geometry(1, 1, 200, 16)
    x = synth.fill(32, synth.T_V, geom, chan_mult=synth.outlier_multipliers(32, 1, 1, 16))
    c1, s1 = oracle.quant_tensor(1, 1, 16, lens, geom.seq_offset, geom.stride_h, geom.stride_t, x)
    c2, s2 = oracle.quant_partitions(1, 1, 16, lens, geom.seq_offset, geom.stride_h, geom.stride_t, x, 200, 1)
    assert s1 == s2[0]
    np.testing.assert_array_equal(c1, c2)


def test_per_tensor_scale_spans_all_heads_and_sequences():
    lens = np.array([5, 9], np.int32)
    geom = synth.packed_token_major_geometry(lens, 3, 8)
    x = np.zeros(geom.numel, np.uint16)
    x[geom.seq_offset[1] + 2 * geom.stride_h + 8 * geom.stride_t + 3] = _bf16([-508.0])[0]
    x[geom.seq_offset[0] + 0 * geom.stride_h + 1 * geom.stride_t + 0] = _bf16([4.0])[0]
    codes, s = oracle.quant_tensor(2, 3, 8, lens, geom.seq_offset, geom.stride_h, geom.stride_t, x)
    assert s == 4.0
    assert codes[geom.seq_offset[1] + 2 * geom.stride_h + 8 * geom.stride_t + 3] == -127
    assert codes[geom.seq_offset[0] + geom.stride_t] == 1


def test_int8_attention_uses_dequantised_values():
    # The oracle's INT8 attention equals fp64 attention on code*scale written out.
    B, KH, G, D, L, part = 1, 2, 4, 32, 150, 64
    q, k, v = random_dense(33, B, KH, G, D, L, fmt=synth.BF16)
    geom = synth.dense_geometry(B, KH, L, D)
    stride = -(-L // part)
    kc, ks = oracle.quant_partitions(B, KH, D, geom.lens, geom.seq_offset, geom.stride_h, geom.stride_t,
                                     k.reshape(-1), part, stride)
    vc, vs = oracle.quant_tensor(B, KH, D, geom.lens, geom.seq_offset, geom.stride_h, geom.stride_t, v.reshape(-1))
    p8 = dense_problem(q, kc.reshape(k.shape), vc.reshape(v.shape))
    p8.k_scale, p8.k_part, p8.k_scale_stride, p8.v_scale = ks, part, stride, vs
    out, lse = oracle.attention_rows(p8, oracle.all_rows(p8))
    kd = kc.reshape(B, KH, L, D).astype(np.float64) * np.repeat(ks.reshape(B, KH, stride), part, axis=2)[:, :, :L, None]
    vd = vc.reshape(B, KH, L, D).astype(np.float64) * np.float64(vs)
    pd = dense_problem(to32(q), kd.astype(np.float32), vd.astype(np.float32))
    # code*scale has at most 32 significant bits, so the float32 copy rounds; compare loosely
    out2, lse2 = oracle.attention_rows(pd, oracle.all_rows(pd))
    np.testing.assert_allclose(out, out2, rtol=0, atol=1e-6)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-6)
    # and it stays close to the unquantised bf16 attention (the page quotes ~0.4% error)
    pb = dense_problem(q, k, v)
    out3, _ = oracle.attention_rows(pb, oracle.all_rows(pb))
    rel = np.linalg.norm(out - out3) / np.linalg.norm(out3)
    assert rel < 0.05


# --- INT8 query (Schemes A/B per-token query partitions, baseline static per-tensor scale) ---


def test_query_rows_and_static_scale_hand_worked(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "int8_query_examples.json")))
    codes, scales = oracle.quant_rows(_bf16(g["rows"]).reshape(-1, g["D"]))
    np.testing.assert_array_equal(codes, np.array(g["row_codes"], np.int8))
    np.testing.assert_array_equal(scales, np.array(g["row_scales"], np.float32))
    sc = oracle.quant_static(_bf16(g["static_values"]), g["static_scale"])
    np.testing.assert_array_equal(sc, np.array(g["static_codes"], np.int8))
    assert not oracle.quant_static(_bf16(g["static_values"]), 0.0).any()


def _query_rows(seed, rows, D):
    q = synth.fill_q(seed, 1, rows, D, synth.BF16).reshape(rows, D).copy()
    q[3, 5] = _bf16([-37.5])[0]   # an outlier row
    q[7] = 0                      # an all-zero row
    return q


@pytest.mark.parametrize("D", [64, 128])
def test_query_rows_max_maps_to_127_and_error_bound(D):
    q = _query_rows(61, 12, D)
    codes, scales = oracle.quant_rows(q)
    qf = to32(q).astype(np.float64)
    assert scales[7] == 0 and not codes[7].any()
    for r in range(12):
        if r == 7:
            continue
        s, cs, vals = np.float64(scales[r]), codes[r].astype(np.int32), qf[r]
        big = np.abs(vals) == np.abs(vals).max()
        assert np.all(cs[big] == np.sign(vals[big]) * 127)
        assert np.all(np.abs(vals - cs * s) <= s * (0.5 + 2.0 ** -17))


def test_query_rows_scale_with_the_row():
    # doubling a row (exact in bf16) doubles its scale exactly and keeps its codes
    q = _query_rows(62, 9, 64)
    q2 = _bf16(to32(q) * np.float32(2.0))
    c1, s1 = oracle.quant_rows(q)
    c2, s2 = oracle.quant_rows(q2)
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_array_equal(s2, s1 * np.float32(2.0))


def test_static_scale_of_a_row_reproduces_its_row_codes():
    q = _query_rows(63, 9, 64)
    codes, scales = oracle.quant_rows(q)
    for r in range(9):
        np.testing.assert_array_equal(oracle.quant_static(q[r], scales[r]), codes[r])
    # a static scale below the row's own clamps the largest values to +-127
    c = oracle.quant_static(q[3], scales[3] / np.float32(4.0))
    big = np.abs(to32(q[3])) >= 127.5 * scales[3] / 4.0
    assert big.any() and np.all(np.abs(c[big]) == 127)


def test_int8_query_attention_uses_the_row_scale():
    # codes with a distinct power-of-two scale per query row: code*scale is exact in fp32, so the
    # int8-query problem must equal the fp32-query problem on those values (a transposed or shifted
    # scale index would not)
    B, KH, G, D, L = 2, 2, 4, 32, 70
    q, k, v = random_dense(64, B, KH, G, D, L, fmt=synth.BF16)
    rows = B * KH * G
    rng = np.random.default_rng(64)
    codes = rng.integers(-127, 128, size=(rows, D)).astype(np.int8)
    qs = (2.0 ** -np.arange(3, 3 + rows)).astype(np.float32)
    p8 = dense_problem(codes.reshape(B, KH * G, D), k, v)
    p8.q_scale = qs
    out8, lse8 = oracle.attention_rows(p8, oracle.all_rows(p8))
    qf = (codes.astype(np.float32) * qs[:, None]).reshape(B, KH * G, D)
    pf = dense_problem(qf, k, v)
    outf, lsef = oracle.attention_rows(pf, oracle.all_rows(pf))
    np.testing.assert_allclose(out8, outf, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse8, lsef, rtol=0, atol=1e-12)
