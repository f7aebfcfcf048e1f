"""Edge cases of the GPU path: empty batches and empty caches, group sizes that need several
column blocks (bf16 and INT8), one-token sequences, lengths at tile and chunk boundaries, the
smallest K partitions, and OAM at its longest sequence (2^21 tokens)."""
import numpy as np
import pytest
import torch

import long_context_decode_gqa_amd as pkg
import oracle
import synth
from gpu_helpers import DEV, dev_geom, log_case, problem, to_dev

pytestmark = pytest.mark.gpu


def test_empty_batch_and_empty_caches():
    log_case("empty batch / empty caches")
    D, KH, G = 128, 2, 8
    empty = pkg.KVGeometry(0, KH, D, 0, torch.zeros(0, dtype=torch.int32, device=DEV),
                           torch.zeros(0, dtype=torch.int64, device=DEV), D, KH * D)
    q0 = torch.zeros((0, KH * G, D), dtype=torch.bfloat16, device=DEV)
    kv0 = torch.zeros(16, dtype=torch.bfloat16, device=DEV)
    out, _ = pkg.attn_decode_splitkv(q0, kv0, kv0, empty, G)
    assert out.shape == (0, KH * G, D)
    # two sequences of length 0: out = 0, lse = -inf; OAM keeps nothing
    lens = torch.zeros(2, dtype=torch.int32, device=DEV)
    geom = pkg.KVGeometry(2, KH, D, 0, lens, torch.zeros(2, dtype=torch.int64, device=DEV), D, KH * D)
    q = torch.randn((2, KH * G, D), device=DEV).to(torch.bfloat16)
    kv = torch.zeros(KH * D, dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros((2, KH * G), dtype=torch.float32, device=DEV)
    out, _ = pkg.attn_decode_splitkv(q, kv, kv, geom, G, lse=lse)
    kc, ks = pkg.kv_quant_int8(kv, geom, 64)
    idx, nk = pkg.oam_score_topk(q, kv, geom, G, 5, v=kv)
    idxb, nkb = pkg.oam_score_topk(q, kv, geom, G, 3, v=kv, block_tokens=64)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))
    assert torch.all(nk == 0) and torch.all(idx == -1)
    assert torch.all(nkb == 0) and torch.all(idxb == -1)


@pytest.mark.parametrize("kv,G", [("bf16", 64), ("bf16", 33), ("int8", 40), ("int8_qrow", 24)])
def test_group_sizes_with_several_column_blocks(kv, G):
    lens = np.array([2500, 17, 1], np.int32)
    w = synth.workload("gqa32k", B=3, KH=2, G=G, D=128, lens=lens, layout="head_major", seed=160 + G)
    q, k, v, g = synth.generate(w)
    log_case(f"group size {G} {kv}")
    qd = to_dev(q.reshape(-1)).view(w.B, w.QH, w.D)
    geom = dev_geom(g)
    lse = torch.empty((w.B, w.QH), dtype=torch.float32, device=DEV)
    pk, qo = {}, q
    if kv == "bf16":
        out, _ = pkg.attn_decode_splitkv(qd, to_dev(k), to_dev(v), geom, G, lse=lse, split_tokens=0)
        kh_, vh_ = k, v
    else:
        kc, ks = pkg.kv_quant_int8(to_dev(k), geom, 64)
        vc, vs = pkg.kv_quant_int8(to_dev(v), geom, 0)
        qq = pkg.QUANT_ROW if kv == "int8_qrow" else pkg.QUANT_EXACT
        out, _ = pkg.attn_decode_splitkv(qd, kc, vc, geom, G, lse=lse, k_scale=ks, k_part_tokens=64,
                                         v_scale=float(vs.item()), q_quant=qq, split_tokens=0)
        torch.cuda.synchronize()
        kh_, vh_ = kc.cpu().numpy(), vc.cpu().numpy()
        pk = dict(k_scale=ks.cpu().numpy(), k_part=64, k_scale_stride=-(-int(g.max_len) // 64),
                  v_scale=float(vs.item()))
        if qq == pkg.QUANT_ROW:
            qc, qs = oracle.quant_rows(q.reshape(-1, w.D))
            qo, pk["q_scale"] = qc.reshape(q.shape), qs
    torch.cuda.synchronize()
    p = problem(w, qo, kh_, vh_, g, **pk)
    ref, ref_lse = oracle.attention_rows(p, oracle.all_rows(p), nthreads=8)
    assert np.abs(out.cpu().numpy().reshape(-1, w.D) - ref).max() <= 2e-3
    assert np.abs(lse.cpu().numpy().reshape(-1) - ref_lse).max() <= 1e-3


def test_many_one_token_sequences_return_their_value():
    B = 300
    lens = np.ones(B, np.int32)
    w = synth.workload("gqa32k", B=B, KH=2, G=8, lens=lens, layout="token_major", seed=170)
    q, k, v, g = synth.generate(w)
    log_case("one-token sequences")
    out, _ = pkg.attn_decode_splitkv(to_dev(q.reshape(-1)).view(w.B, w.QH, w.D), to_dev(k), to_dev(v), dev_geom(g),
                                     w.G, split_tokens=0)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    vf = synth.bf16_bits_to_f32(v)
    for b in range(0, B, 37):
        for kh in range(w.KH):
            row = vf[g.seq_offset[b] + kh * g.stride_h:][:w.D]
            assert np.abs(out[b, kh * w.G:(kh + 1) * w.G] - row[None, :]).max() <= 1e-6


@pytest.mark.parametrize("kind", ["bf16", "int8", "indexed"])
def test_more_lanes_than_a_worker_stages(kind):
    """70 sequences x 4 KV heads = 280 (b, kh) lanes, more than the 256 whose lengths a decode
    worker stages in LDS at its start: the work split and the lane walk then read the lengths and
    offsets from global memory.  Ragged lengths with empty sequences; every output row and lse
    against the oracle, on a bf16 cache, an INT8 cache, and a kept-token list per lane."""
    rng = np.random.default_rng(175)
    lens = rng.integers(1, 700, 70).astype(np.int32)
    lens[::9] = 0
    lens[5] = 4000
    w = synth.workload("gqa32k", B=70, KH=4, G=8, lens=lens, layout="token_major", seed=175)
    q, k, v, g = synth.generate(w)
    log_case(f"280 lanes, {kind}")
    qd = to_dev(q.reshape(-1)).view(w.B, w.QH, w.D)
    geom = dev_geom(g)
    lse = torch.empty((w.B, w.QH), dtype=torch.float32, device=DEV)
    pk, kh_, vh_ = {}, k, v
    kw = dict(lse=lse, split_tokens=256)
    if kind == "int8":
        kc, ks = pkg.kv_quant_int8(to_dev(k), geom, 64)
        vc, vs = pkg.kv_quant_int8(to_dev(v), geom, 0)
        torch.cuda.synchronize()
        out, _ = pkg.attn_decode_splitkv(qd, kc, vc, geom, w.G, k_scale=ks, k_part_tokens=64,
                                         v_scale=float(vs.item()), **kw)
        kh_, vh_ = kc.cpu().numpy(), vc.cpu().numpy()
        pk = dict(k_scale=ks.cpu().numpy(), k_part=64, k_scale_stride=-(-int(g.max_len) // 64),
                  v_scale=float(vs.item()))
    else:
        if kind == "indexed":
            stride = 300
            idx = np.full((w.B * w.KH, stride), -1, np.int32)
            nk = np.zeros(w.B * w.KH, np.int32)
            for pr in range(w.B * w.KH):
                L = int(lens[pr // w.KH])
                n = min(L, int(rng.integers(0, stride + 1)))
                idx[pr, :n] = np.sort(rng.choice(L, n, replace=False)) if n else idx[pr, :0]
                nk[pr] = n
            kw.update(token_idx=to_dev(idx), n_idx=to_dev(nk))
            pk = dict(tok_idx=idx.reshape(-1), n_idx=nk, idx_stride=stride)
        out, _ = pkg.attn_decode_splitkv(qd, to_dev(k), to_dev(v), geom, w.G, **kw)
    torch.cuda.synchronize()
    p = problem(w, q, kh_, vh_, g, **pk)
    ref, ref_lse = oracle.attention_rows(p, oracle.all_rows(p), nthreads=8)
    assert np.abs(out.cpu().numpy().reshape(-1, w.D) - ref).max() <= 2e-3
    got_lse = lse.cpu().numpy().reshape(-1)
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(got_lse), empty)
    assert np.abs(got_lse[~empty] - ref_lse[~empty]).max() <= 1e-3


@pytest.mark.parametrize("split", [0, 64, 2048])
def test_lengths_at_tile_and_chunk_boundaries(split):
    lens = np.array([31, 32, 33, 63, 64, 65, 2047, 2048, 2049, 4096], np.int32)
    w = synth.workload("gqa32k", B=len(lens), KH=1, G=8, lens=lens, layout="token_major", seed=171)
    q, k, v, g = synth.generate(w)
    log_case(f"boundary lengths split={split}")
    lse = torch.empty((w.B, w.QH), dtype=torch.float32, device=DEV)
    out, _ = pkg.attn_decode_splitkv(to_dev(q.reshape(-1)).view(w.B, w.QH, w.D), to_dev(k), to_dev(v), dev_geom(g),
                                     w.G, lse=lse, split_tokens=split)
    torch.cuda.synchronize()
    p = problem(w, q, k, v, g)
    ref, ref_lse = oracle.attention_rows(p, oracle.all_rows(p), nthreads=8)
    assert np.abs(out.cpu().numpy().reshape(-1, w.D) - ref).max() <= 2e-3
    assert np.abs(lse.cpu().numpy().reshape(-1) - ref_lse).max() <= 1e-3


def test_int8_smallest_partitions():
    lens = np.array([700, 33], np.int32)
    w = synth.workload("int8_128k", B=2, KH=2, G=8, lens=lens, layout="token_major", seed=172)
    q, k, v, g = synth.generate(w)
    log_case("int8 16-token partitions")
    geom = dev_geom(g)
    kc, ks = pkg.kv_quant_int8(to_dev(k), geom, 16)
    vc, vs = pkg.kv_quant_int8(to_dev(v), geom, 0)
    out, _ = pkg.attn_decode_splitkv(to_dev(q.reshape(-1)).view(w.B, w.QH, w.D), kc, vc, geom, w.G, k_scale=ks,
                                     k_part_tokens=16, v_scale=float(vs.item()), split_tokens=0)
    torch.cuda.synchronize()
    p = problem(w, q, kc.cpu().numpy(), vc.cpu().numpy(), g, k_scale=ks.cpu().numpy(), k_part=16,
                k_scale_stride=-(-700 // 16), v_scale=float(vs.item()))
    ref, _ = oracle.attention_rows(p, oracle.all_rows(p), nthreads=8)
    assert np.abs(out.cpu().numpy().reshape(-1, w.D) - ref).max() <= 2e-3


def test_oam_at_the_longest_sequence():
    """One (sequence, KV head) of 2^21 tokens, the most the selection supports (1024 blocks of
    2048 tokens), G = 1: kept set against the oracle within the score band."""
    L = 1 << 21
    w = synth.workload("oam_128k", B=1, KH=1, G=1, lens=np.array([L], np.int32), seed=173)
    q, k, v, g = synth.generate(w)
    log_case("oam 2^21 tokens")
    qd = to_dev(q.reshape(-1)).view(1, 1, w.D)
    kd, vd = to_dev(k), to_dev(v)
    scores = torch.empty((1, L), dtype=torch.float32, device=DEV)
    idx, nk = pkg.oam_score_topk(qd, kd, dev_geom(g), 1, 4096, v=vd, scores_out=scores)
    torch.cuda.synchronize()
    p = problem(w, q, k, v, g)
    ref_s = oracle.oam_scores(p, 0, 0, 1.0, 1e-6)
    gpu_s = scores.cpu().numpy()[0]
    assert np.abs(gpu_s - ref_s).max() <= 5e-5
    kept = idx.cpu().numpy()[0, :int(nk.cpu().numpy()[0])]
    assert len(kept) == 4096 and np.all(np.diff(kept) > 0)
    order = np.lexsort((np.arange(L), -gpu_s.astype(np.float64)))
    np.testing.assert_array_equal(kept, np.sort(order[:4096]))
    ref = oracle.topk_sort(ref_s, 4096)
    thr = np.sort(ref_s)[::-1][4095]
    assert all(abs(ref_s[i] - thr) <= 1e-4 for i in set(kept.tolist()) ^ set(ref.tolist()))
