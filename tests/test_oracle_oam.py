"""Pins of the oracle's output-aware token dropping (OAM).

Source: "优化稀疏注意力中的令牌丢弃机制" §2 (classic q.k/sqrt(d_k) top-K), §3 (OAM
pseudo-code: routing score q.k_i/sqrt(d_k) plus beta*log(||v_i|| + eps); drop the
lowest scores).  Readings: mean over the G query heads of a KV head, ties to the
lower index, K >= L keeps everything.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth
from helpers import dense_problem, random_dense, with_tokens


def _hand_problem(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "oam_hand_example.json")))
    D, G = g["D"], g["G"]
    q = np.array(g["q"], np.float32).reshape(1, G, D)
    k = np.array(g["k"], np.float32).reshape(1, 1, -1, D)
    v = np.array(g["v"], np.float32).reshape(1, 1, -1, D)
    return g, dense_problem(q, k, v, softmax_scale=g["softmax_scale"])


def test_hand_worked_scores_and_selection(golden_dir):
    g, p = _hand_problem(golden_dir)
    s = oracle.oam_scores(p, 0, 0, g["beta"], g["eps"])
    np.testing.assert_allclose(s, g["scores"], rtol=0, atol=g["tol"])
    for k, want in g["topk"].items():
        assert list(oracle.topk_sort(s, int(k))) == want
        assert list(oracle.topk_select(s, int(k))) == want
    s0 = oracle.oam_scores(p, 0, 0, 0.0, g["eps"])
    for k, want in g["topk_beta0"].items():
        assert list(oracle.topk_sort(s0, int(k))) == want


def test_value_lognorm_closed_form(golden_dir):
    g, p = _hand_problem(golden_dir)
    vl = oracle.value_lognorm(p, 0, 0, 1e-6)
    np.testing.assert_allclose(vl, [math.log(5 + 1e-6), math.log(1 + 1e-6), math.log(10 + 1e-6),
                                    math.log(0.5 + 1e-6)], rtol=0, atol=1e-15)


def test_beta_zero_is_classic_mean_qk_ranking():
    B, KH, G, D, L = 1, 2, 4, 32, 500
    q, k, v = random_dense(41, B, KH, G, D, L)
    p = dense_problem(q, k, v)
    for kh in range(KH):
        s = oracle.oam_scores(p, 0, kh, 0.0, 1e-6)
        ref = (k[0, kh].astype(np.float64) @ q[0, kh * G:(kh + 1) * G].astype(np.float64).T).mean(axis=1) / math.sqrt(D)
        np.testing.assert_allclose(s, ref, rtol=1e-12, atol=1e-13)
        order = np.lexsort((np.arange(L), -ref))[:37]
        assert list(oracle.topk_sort(s, 37)) == sorted(order.tolist())


def test_value_term_is_log_of_l2_norm():
    B, KH, G, D, L = 1, 1, 2, 16, 50
    q, k, v = random_dense(42, B, KH, G, D, L)
    p = dense_problem(q, k, v)
    s1 = oracle.oam_scores(p, 0, 0, 1.0, 1e-6)
    s0 = oracle.oam_scores(p, 0, 0, 0.0, 1e-6)
    np.testing.assert_allclose(s1 - s0, np.log(np.linalg.norm(v[0, 0].astype(np.float64), axis=1) + 1e-6),
                               rtol=0, atol=1e-13)
    s2 = oracle.oam_scores(p, 0, 0, 2.5, 1e-6)
    np.testing.assert_allclose(s2 - s0, 2.5 * (s1 - s0), rtol=0, atol=1e-13)


def test_constant_scores_keep_lowest_indices():
    s = np.full(1000, 0.25)
    assert list(oracle.topk_sort(s, 10)) == list(range(10))
    assert list(oracle.topk_select(s, 10)) == list(range(10))


@pytest.mark.parametrize("k", [1, 5, 100, 999, 1000, 5000])
def test_sort_and_select_forms_agree_with_ties(k):
    rng = np.random.default_rng(k)
    s = rng.integers(0, 20, size=1000).astype(np.float64)   # many ties
    a = oracle.topk_sort(s, k)
    b = oracle.topk_select(s, k)
    np.testing.assert_array_equal(a, b)
    assert len(a) == min(k, 1000) and np.all(np.diff(a) > 0)
    if 0 < k < 1000:
        thr = np.sort(s)[::-1][k - 1]
        assert np.all(s[a] >= thr) and np.sum(s > thr) <= k
        kept = set(a.tolist())
        # every dropped token scores below the threshold, or ties it with a higher index
        for i in range(1000):
            if i not in kept:
                assert s[i] < thr or (s[i] == thr and i > max(j for j in kept if s[j] == thr))


def test_keep_all_reduces_to_dense_attention():
    B, KH, G, D, L = 1, 2, 4, 32, 200
    q, k, v = random_dense(43, B, KH, G, D, L)
    p = dense_problem(q, k, v)
    out, lse = oracle.attention_rows(p, oracle.all_rows(p))
    idx = [oracle.topk_sort(oracle.oam_scores(p, 0, kh, 1.0, 1e-6), 4096) for kh in range(KH)]
    assert all(len(x) == L for x in idx)
    out2, lse2 = oracle.attention_rows(with_tokens(p, idx), oracle.all_rows(p))
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


def test_one_dominant_token_with_k1_returns_its_value():
    B, KH, G, D, L = 1, 1, 2, 16, 64
    q, k, v = random_dense(44, B, KH, G, D, L)
    v[0, 0, 17] *= 1e6      # huge value norm dominates the OAM score
    p = dense_problem(q, k, v)
    s = oracle.oam_scores(p, 0, 0, 1.0, 1e-6)
    idx = oracle.topk_sort(s, 1)
    assert list(idx) == [17]
    out, _ = oracle.attention_rows(with_tokens(p, [idx]), oracle.all_rows(p))
    np.testing.assert_allclose(out, np.broadcast_to(v[0, 0, 17].astype(np.float64), out.shape), rtol=0, atol=1e-9)


def test_oam_over_an_int8_cache_uses_the_dequantised_values():
    """The page's §7 stack: OAM over an INT8 cache scores the values the attention reads, code x
    scale.  With power-of-two K partition scales and V scale, code x scale is exact in fp32, so the
    INT8 problem's scores and value terms equal those of the fp32 problem on those values (a wrong
    partition index or a missing V scale would not)."""
    B, KH, G, D, L, part = 2, 2, 4, 32, 200, 64
    rng = np.random.default_rng(81)
    geom = synth.dense_geometry(B, KH, L, D)
    kc = rng.integers(-127, 128, size=(B, KH, L, D)).astype(np.int8)
    vc = rng.integers(-127, 128, size=(B, KH, L, D)).astype(np.int8)
    stride = -(-L // part)
    ks = (2.0 ** -rng.integers(3, 9, size=B * KH * stride)).astype(np.float32)
    vs = np.float32(2.0 ** -6)
    q = synth.fill_q(81, B, KH * G, D, synth.BF16)
    p8 = dense_problem(q, kc, vc)
    p8.k_scale, p8.k_part, p8.k_scale_stride, p8.v_scale = ks, part, stride, float(vs)
    kf = kc.astype(np.float32) * np.repeat(ks.reshape(B, KH, stride), part, axis=2)[:, :, :L, None]
    vf = vc.astype(np.float32) * vs
    pf = dense_problem(q, kf, vf)
    for b in range(B):
        for kh in range(KH):
            np.testing.assert_allclose(oracle.value_lognorm(p8, b, kh, 1e-6), oracle.value_lognorm(pf, b, kh, 1e-6),
                                       rtol=0, atol=1e-12)
            s8 = oracle.oam_scores(p8, b, kh, 1.0, 1e-6)
            np.testing.assert_allclose(s8, oracle.oam_scores(pf, b, kh, 1.0, 1e-6), rtol=0, atol=1e-12)
            assert list(oracle.topk_sort(s8, 37)) == list(oracle.topk_sort(oracle.oam_scores(pf, b, kh, 1.0, 1e-6), 37))
