"""Pins of the oracle's block-granular selection.

Source: "原生稀疏注意力(NSA)" §2.1, selected attention: top-n blocks of contiguous tokens
(64 on the page) by an importance shared by the GQA group; the learned block compression
read as the mean over the block (so a block's score is the mean of its tokens' scores).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth
from helpers import dense_problem, random_dense


def _line_problem(s):
    L = len(s)
    q = np.array([1.0, 0.0], np.float32).reshape(1, 1, 2)
    k = np.zeros((1, 1, L, 2), np.float32)
    k[0, 0, :, 0] = s
    v = np.ones((1, 1, L, 2), np.float32)
    return dense_problem(q, k, v, softmax_scale=1.0)


def test_hand_worked_block_scores_and_kept_tokens(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "block_select_hand_example.json")))
    for case in g["cases"]:
        p = _line_problem(case["s"])
        for n, want in case["kept"].items():
            idx, bs = oracle.block_select(p, 0, 0, g["block_tokens"], int(n), beta=0.0)
            assert list(idx) == want
            np.testing.assert_allclose(bs, case["block_scores"], rtol=0, atol=1e-12)


@pytest.mark.parametrize("beta", [0.0, 1.0])
def test_one_token_blocks_are_the_token_top_k(beta):
    q, k, v = random_dense(71, 1, 2, 4, 32, 300, fmt=synth.BF16)
    p = dense_problem(q, k, v)
    for kh in range(2):
        idx, _ = oracle.block_select(p, 0, kh, 1, 37, beta=beta)
        want = oracle.topk_sort(oracle.oam_scores(p, 0, kh, beta, 1e-6), 37)
        np.testing.assert_array_equal(idx, want)


def test_block_score_is_the_query_against_the_mean_key():
    # mean pooling as the block compression: by linearity the mean of the blocks' token scores
    # equals the group's mean query against the block's mean key
    B, KH, G, D, L, bt = 1, 2, 4, 16, 150, 64
    q, k, v = random_dense(72, B, KH, G, D, L, fmt=synth.F32)
    p = dense_problem(q, k, v)
    for kh in range(KH):
        _, bs = oracle.block_select(p, 0, kh, bt, 1, beta=0.0)
        qbar = q[0, kh * G:(kh + 1) * G].astype(np.float64).mean(axis=0)
        for j in range(len(bs)):
            kbar = k[0, kh, j * bt:min(L, (j + 1) * bt)].astype(np.float64).mean(axis=0)
            assert abs(bs[j] - qbar @ kbar / math.sqrt(D)) <= 1e-12


def test_keeping_every_block_is_dense_attention():
    lens = np.array([200, 64, 1], np.int32)
    w = synth.workload("gqa32k", B=3, KH=2, G=4, D=32, lens=lens, layout="token_major", seed=73)
    q, k, v, g = synth.generate(w)
    p = oracle.Problem(w.B, w.KH, w.G, w.D, g.lens, g.seq_offset, g.stride_h, g.stride_t, q, k, v,
                       1.0 / math.sqrt(w.D))
    lists = []
    for b in range(w.B):
        for kh in range(w.KH):
            idx, _ = oracle.block_select(p, b, kh, 64, 10, beta=0.0)
            np.testing.assert_array_equal(idx, np.arange(lens[b]))
            lists.append(idx)
    from helpers import with_tokens
    out_k, _ = oracle.attention_rows(with_tokens(p, lists), oracle.all_rows(p))
    out_d, _ = oracle.attention_rows(p, oracle.all_rows(p))
    np.testing.assert_allclose(out_k, out_d, rtol=0, atol=1e-12)


def test_kept_blocks_are_whole_and_ascending():
    q, k, v = random_dense(74, 1, 1, 8, 32, 1000, fmt=synth.BF16)
    p = dense_problem(q, k, v)
    idx, bs = oracle.block_select(p, 0, 0, 64, 5, beta=0.0)
    assert np.all(np.diff(idx) > 0)
    blocks = sorted(set((idx // 64).tolist()))
    assert len(blocks) == 5
    sizes = [min(1000, (j + 1) * 64) - j * 64 for j in blocks]
    assert len(idx) == sum(sizes)
    # every kept block scores at least as high as every dropped one
    dropped = [j for j in range(len(bs)) if j not in blocks]
    assert min(bs[blocks]) >= max(bs[dropped])
