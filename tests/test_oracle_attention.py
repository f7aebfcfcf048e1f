"""Pins of the oracle's attention, partial and merge functions.

Each test checks the oracle against something other than itself: values
worked by hand (tests/golden), closed forms, invariances the definition
implies, a second independent formulation, or a library routine on a special
case.  Sources: softmax(QK^T/sqrt(d_k))V on "注意力优化（Attention Optimization）";
out = sum_i softmax(q.k_i/sqrt(d)) v_i and the cross-shard online softmax of
"优化稀疏注意力中的令牌丢弃机制" §2 and §5; the GQA repeat_interleave example on
"注意力优化（Attention Optimization）" (运行示例).
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle
import synth
from helpers import dense_problem, random_dense, with_tokens


def _golden(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def test_hand_worked_examples(golden_dir):
    g = _golden(golden_dir, "attention_hand_examples.json")
    for case in g["cases"]:
        D, G = case["D"], case["G"]
        q = np.array(case["q"], np.float32).reshape(1, G, D)
        k = np.array(case["k"], np.float32).reshape(1, 1, -1, D)
        v = np.array(case["v"], np.float32).reshape(1, 1, -1, D)
        p = dense_problem(q, k, v, softmax_scale=case["softmax_scale"])
        for form in ("plain", "online"):
            if form == "plain":
                out, lse = oracle.attention_rows(p, oracle.all_rows(p))
            else:
                out, lse = oracle.attention_rows_online(p, oracle.all_rows(p), 1)
            np.testing.assert_allclose(out, np.array(case["out"]), atol=case["tol"], rtol=0, err_msg=case["name"])
            np.testing.assert_allclose(lse, np.array(case["lse"]), atol=case["tol"], rtol=0, err_msg=case["name"])


def test_single_token_returns_its_value():
    q, k, v = random_dense(11, 2, 2, 3, 16, 1)
    p = dense_problem(q, k, v)
    out, lse = oracle.attention_rows(p, oracle.all_rows(p))
    for r, (b, qh) in enumerate(oracle.all_rows(p)):
        kh = qh // 3
        np.testing.assert_allclose(out[r], v[b, kh, 0].astype(np.float64), rtol=0, atol=1e-15)
        s = float(np.dot(q[b, qh].astype(np.float64), k[b, kh, 0].astype(np.float64))) / 4.0
        assert abs(lse[r] - s) < 1e-12


def test_constant_value_returns_it():
    q, k, _ = random_dense(12, 1, 2, 4, 32, 300)
    v = np.broadcast_to(np.linspace(-2, 3, 32, dtype=np.float32), (1, 2, 300, 32)).copy()
    p = dense_problem(q, k, v)
    out, _ = oracle.attention_rows(p, oracle.all_rows(p))
    np.testing.assert_allclose(out, np.broadcast_to(v[0, 0, 0], out.shape), rtol=0, atol=1e-13)


def test_zero_query_is_mean_of_values():
    _, k, v = random_dense(13, 1, 1, 2, 16, 257)
    q = np.zeros((1, 2, 16), np.float32)
    p = dense_problem(q, k, v)
    out, lse = oracle.attention_rows(p, oracle.all_rows(p))
    np.testing.assert_allclose(out[0], v[0, 0].astype(np.float64).mean(axis=0), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, [math.log(257)] * 2, rtol=0, atol=1e-13)


def test_matches_library_softmax_brute_force():
    # scipy's softmax/logsumexp on the whole score vector: the textbook form.
    q, k, v = random_dense(14, 2, 2, 4, 64, 97)
    p = dense_problem(q, k, v)
    out, lse = oracle.attention_rows(p, oracle.all_rows(p))
    for r, (b, qh) in enumerate(oracle.all_rows(p)):
        kh = qh // 4
        s = k[b, kh].astype(np.float64) @ q[b, qh].astype(np.float64) / 8.0
        np.testing.assert_allclose(out[r], softmax(s) @ v[b, kh].astype(np.float64), rtol=1e-12, atol=1e-13)
        assert abs(lse[r] - logsumexp(s)) < 1e-12


def test_gqa_equals_mha_on_repeated_kv():
    # GQA reads KV head qh // G; repeating each KV head G times gives MHA.
    G = 4
    q, k, v = random_dense(15, 2, 2, G, 32, 65)
    p = dense_problem(q, k, v)
    out, lse = oracle.attention_rows(p, oracle.all_rows(p))
    k_rep = np.repeat(k, G, axis=1)
    v_rep = np.repeat(v, G, axis=1)
    p_mha = dense_problem(q, k_rep, v_rep)
    assert p_mha.G == 1
    out2, lse2 = oracle.attention_rows(p_mha, oracle.all_rows(p_mha))
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


def test_head_mapping_groups_consecutive_query_heads():
    # Only KV head 1 carries non-zero values: query heads G..2G-1 must see them.
    G = 3
    q, k, v = random_dense(16, 1, 2, G, 8, 10)
    v[0, 0] = 0.0
    p = dense_problem(q, k, v)
    out, _ = oracle.attention_rows(p, oracle.all_rows(p))
    assert np.all(out[:G] == 0.0)
    assert np.all(np.abs(out[G:]).sum(axis=1) > 0)


def test_token_permutation_invariance():
    q, k, v = random_dense(17, 1, 2, 2, 16, 50)
    p = dense_problem(q, k, v)
    out, lse = oracle.attention_rows(p, oracle.all_rows(p))
    rng = np.random.default_rng(0)
    perm = [list(rng.permutation(50)) for _ in range(2)]
    out2, lse2 = oracle.attention_rows(with_tokens(p, perm), oracle.all_rows(p))
    np.testing.assert_allclose(out2, out, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, rtol=1e-14, atol=0)


@pytest.mark.parametrize("block", [1, 7, 64, 1000])
def test_online_form_agrees_with_plain_definition(block):
    q, k, v = random_dense(18, 2, 2, 4, 64, 333)
    p = dense_problem(q, k, v)
    out, lse = oracle.attention_rows(p, oracle.all_rows(p))
    out2, lse2 = oracle.attention_rows_online(p, oracle.all_rows(p), block)
    np.testing.assert_allclose(out2, out, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=1e-12, atol=0)


@pytest.mark.parametrize("cuts", [[0, 333], [0, 1, 333], [0, 100, 100, 200, 333], [0, 256, 332, 333],
                                  list(range(0, 334, 1))[:40] + [333]])
def test_split_then_merge_equals_unsplit(cuts):
    q, k, v = random_dense(19, 1, 1, 4, 64, 333)
    p = dense_problem(q, k, v)
    out, lse = oracle.attention_rows(p, oracle.all_rows(p))
    for qh in range(4):
        parts = [oracle.partial(p, 0, qh, a, b) for a, b in zip(cuts[:-1], cuts[1:])]
        m = np.array([x[0] for x in parts])
        l = np.array([x[1] for x in parts])
        o = np.stack([x[2] for x in parts])
        mo, ml = oracle.merge(m, l, o)
        np.testing.assert_allclose(mo, out[qh], rtol=1e-12, atol=1e-13)
        assert abs(ml - lse[qh]) <= 1e-12 * abs(lse[qh])


def test_merge_weights_each_chunk_by_its_own_max():
    # A merge that forgets exp(m_chunk - m_new) on the chunk term fails here:
    # two one-token chunks with scores 0 and ln 3 must weigh 1/4 and 3/4.
    m = np.array([0.0, math.log(3.0)])
    l = np.array([1.0, 1.0])
    o = np.array([[1.0, 0.0], [0.0, 1.0]])
    out, lse = oracle.merge(m, l, o)
    np.testing.assert_allclose(out, [0.25, 0.75], rtol=0, atol=1e-15)
    assert abs(lse - math.log(4.0)) < 1e-15
    out2, lse2 = oracle.merge(m[::-1].copy(), l[::-1].copy(), o[::-1].copy())
    np.testing.assert_allclose(out2, out, rtol=0, atol=1e-15)


def test_empty_inputs():
    q, k, v = random_dense(20, 2, 1, 2, 16, 8)
    p = dense_problem(q, k, v, lens=[0, 8])
    out, lse = oracle.attention_rows(p, oracle.all_rows(p))
    assert np.all(out[:2] == 0.0) and np.all(np.isneginf(lse[:2]))
    assert np.all(np.isfinite(lse[2:]))
    m, l, o = oracle.partial(p, 1, 0, 3, 3)
    assert m == -math.inf and l == 0.0 and np.all(o == 0.0)
    out2, lse2 = oracle.merge(np.array([-math.inf]), np.array([0.0]), np.zeros((1, 16)))
    assert np.all(out2 == 0.0) and lse2 == -math.inf


def test_bf16_inputs_are_read_exactly():
    # bf16 bit patterns widen exactly: same problem as float32 gives the same result.
    q, k, v = random_dense(21, 1, 2, 2, 32, 40, fmt=1)
    to32 = lambda a: (a.astype(np.uint32) << 16).view(np.float32)
    p16 = dense_problem(q, k, v)
    p32 = dense_problem(to32(q), to32(k), to32(v))
    a = oracle.attention_rows(p16, oracle.all_rows(p16))
    b = oracle.attention_rows(p32, oracle.all_rows(p32))
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


# --- multi-row (speculative) decode: the NV blog's (1 + draft) x G GEMM-M ---


def test_multirow_hand_worked(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "multirow_hand_example.json")))
    L, R, D = g["L"], g["R"], g["D"]
    q = np.zeros((1, R, 1, D), np.float32)
    k = np.array([[1.0, 2.0], [-4.0, 0.5], [7.0, 7.0]], np.float32).reshape(1, 1, L, D)
    v = np.array(g["v"], np.float32).reshape(1, 1, L, D)
    p = dense_problem(np.ascontiguousarray(q[:, 0]), k, v)   # G = 1 query head per KV head
    p.q = q
    out, lse = oracle.attention_multirow(p, R, [(0, 0, 0), (0, 1, 0)])
    np.testing.assert_allclose(out, g["out"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, g["lse"], rtol=0, atol=1e-12)


def test_multirow_one_row_is_plain_decode_and_last_row_sees_everything():
    B, KH, G, D, L, R = 2, 2, 4, 32, 90, 3
    q, k, v = random_dense(75, B, KH, G * R, D, L, fmt=synth.BF16)  # q values reshaped to [B, R, KH*G, D]
    qr = np.ascontiguousarray(q.reshape(B, R, KH * G, D))
    p = dense_problem(np.ascontiguousarray(qr[:, 0]), k, v)
    p.q = qr
    rows = [(b, r, qh) for b in range(B) for r in range(R) for qh in range(KH * G)]
    out, lse = oracle.attention_multirow(p, R, rows)
    # the last row attends to the whole cache: the plain definition with that row's query
    plast = dense_problem(np.ascontiguousarray(qr[:, R - 1]), k, v)
    o2, l2 = oracle.attention_rows(plast, oracle.all_rows(plast))
    last = [i for i, r in enumerate(rows) if r[1] == R - 1]
    np.testing.assert_allclose(out[last], o2, rtol=0, atol=1e-12)
    # one row: identical to attention_rows
    p1 = dense_problem(np.ascontiguousarray(qr[:, 0]), k, v)
    o1, l1 = oracle.attention_multirow(p1, 1, [(b, 0, qh) for b in range(B) for qh in range(KH * G)])
    o0, l0 = oracle.attention_rows(p1, oracle.all_rows(p1))
    np.testing.assert_array_equal(o1, o0)
    # row r sees the first L - (R - 1) + r tokens: the same row over a cache cut to that prefix and
    # asked as the last of R rows gives the same result
    for r in range(R - 1):
        cut = L - (R - 1) + r
        pc = dense_problem(np.ascontiguousarray(qr[:, 0]), np.ascontiguousarray(k[:, :, :cut]),
                           np.ascontiguousarray(v[:, :, :cut]))
        pc.q = np.ascontiguousarray(np.concatenate([qr[:, r:r + 1]] * R, axis=1))
        oc, _ = oracle.attention_multirow(pc, R, [(b, R - 1, qh) for b in range(B) for qh in range(KH * G)])
        rr = [i for i, x in enumerate(rows) if x[1] == r]
        np.testing.assert_allclose(out[rr], oc, rtol=0, atol=1e-12)
