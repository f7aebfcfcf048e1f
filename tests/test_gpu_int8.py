"""GPU parity of kv_quant_int8 (bit-exact codes and scales) and INT8-KV decode.

Codes and scales must equal the oracle's fp32 definition bit for bit; INT8
decode outputs are compared with the fp64 oracle over the same dequantised
values within 2e-3 max-abs.
"""
import math

import numpy as np
import pytest
import torch

import long_context_decode_gqa_amd as pkg
import oracle
import synth
from gpu_helpers import DEV, dev_geom, log_case, problem, to_dev

pytestmark = pytest.mark.gpu


def gen_kv(w):
    q, k, v, g = synth.generate(w)
    return q, k, v, g


def gpu_quant(x16, g, part):
    codes, scales = pkg.kv_quant_int8(to_dev(x16), dev_geom(g), part)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


@pytest.mark.parametrize("part", [64, 128, 16])
def test_partition_quant_bit_exact_ragged(part):
    lens = np.array([1, 63, 64, 65, 700, 2049, 0, 130], np.int32)
    w = synth.workload("int8_128k", B=len(lens), KH=3, lens=lens, layout="token_major", seed=40 + part)
    q, k, v, g = gen_kv(w)
    log_case(f"int8 partition quant part={part}")
    stride = max(1, -(-int(lens.max()) // part))
    ref_codes, ref_scales = oracle.quant_partitions(g.B, g.KH, g.D, g.lens, g.seq_offset, g.stride_h, g.stride_t,
                                                    k, part, stride)
    codes, scales = gpu_quant(k, g, part)
    # compare only written rows / partitions
    mask = np.zeros(g.numel, bool)
    for b in range(g.B):
        for kh in range(g.KH):
            for t in range(lens[b]):
                o = g.seq_offset[b] + kh * g.stride_h + t * g.stride_t
                mask[o:o + g.D] = True
    np.testing.assert_array_equal(codes[mask], ref_codes[mask])
    for b in range(g.B):
        for kh in range(g.KH):
            n = -(-int(lens[b]) // part)
            base = (b * g.KH + kh) * stride
            np.testing.assert_array_equal(scales[base:base + n], ref_scales[base:base + n])


def test_tensor_quant_bit_exact_and_zero_partitions():
    lens = np.array([300, 5, 129], np.int32)
    w = synth.workload("int8_128k", B=3, KH=2, lens=lens, layout="head_major", seed=47)
    q, k, v, g = gen_kv(w)
    # an all-zero 64-token partition must give scale 0 and codes 0
    for t in range(64, 128):
        o = g.seq_offset[0] + 1 * g.stride_h + t * g.stride_t
        k[o:o + g.D] = 0
    log_case("int8 per-tensor quant")
    ref_codes, ref_scale = oracle.quant_tensor(g.B, g.KH, g.D, g.lens, g.seq_offset, g.stride_h, g.stride_t, v)
    codes, scales = gpu_quant(v, g, 0)
    assert scales[0] == np.float32(ref_scale)
    np.testing.assert_array_equal(codes, ref_codes)
    ref_k, ref_ks = oracle.quant_partitions(g.B, g.KH, g.D, g.lens, g.seq_offset, g.stride_h, g.stride_t, k, 64, 5)
    kc, ks = gpu_quant(k, g, 64)
    np.testing.assert_array_equal(kc, ref_k)
    np.testing.assert_array_equal(ks, ref_ks)
    assert ks[(0 * g.KH + 1) * 5 + 1] == 0.0


def run_int8_decode(w, q, kc, vc, ks, vs, g, part=64, token_idx=None, n_idx=None, split=1024):
    qd = to_dev(q.reshape(-1)).view(w.B, w.QH, w.D)
    lse = torch.empty((w.B, w.QH), dtype=torch.float32, device=DEV)
    kw = {}
    if token_idx is not None:
        kw = dict(token_idx=to_dev(token_idx), n_idx=to_dev(n_idx))
    out, _ = pkg.attn_decode_splitkv(qd, to_dev(kc), to_dev(vc), dev_geom(g), w.G, lse=lse, k_scale=to_dev(ks),
                                     k_part_tokens=part, v_scale=float(vs), split_tokens=split, **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy().reshape(w.B * w.QH, w.D), lse.cpu().numpy().reshape(-1)


@pytest.mark.parametrize("G,D", [(8, 128), (4, 64), (16, 128)])
def test_int8_decode_matches_oracle_on_dequantised_values(G, D):
    lens = np.array([3000, 1, 64, 1500], np.int32)
    w = synth.workload("int8_128k", B=4, KH=2, G=G, D=D, lens=lens, layout="token_major", seed=50 + G)
    q, k, v, g = gen_kv(w)
    log_case(f"int8 decode G={G} D={D}")
    stride = -(-int(lens.max()) // 64)
    kc, ks = gpu_quant(k, g, 64)
    vc, vsa = gpu_quant(v, g, 0)
    p = problem(w, q, kc, vc, g, k_scale=ks, k_part=64, k_scale_stride=stride, v_scale=float(vsa[0]))
    ref, ref_lse = oracle.attention_rows(p, oracle.all_rows(p), nthreads=8)
    for split in (1024, 256, 0):
        out, lse = run_int8_decode(w, q, kc, vc, ks, vsa[0], g, split=split)
        assert np.abs(out - ref).max() <= 2e-3
        assert np.abs(lse - ref_lse).max() <= 1e-3


def test_int8_decode_with_kept_token_subset():
    lens = np.array([2000, 900], np.int32)
    w = synth.workload("int8_128k", B=2, KH=2, G=8, lens=lens, layout="token_major", seed=58)
    q, k, v, g = gen_kv(w)
    kc, ks = gpu_quant(k, g, 64)
    vc, vsa = gpu_quant(v, g, 0)
    rng = np.random.default_rng(5)
    stride = 600
    idx = np.zeros((4, stride), np.int32)
    nidx = np.array([600, 17, 300, 1], np.int32)
    for i in range(4):
        idx[i, :nidx[i]] = np.sort(rng.choice(lens[i // 2], size=nidx[i], replace=False))
    log_case("int8 decode kept subset")
    p = problem(w, q, kc, vc, g, k_scale=ks, k_part=64, k_scale_stride=-(-2000 // 64), v_scale=float(vsa[0]),
                tok_idx=idx.reshape(-1), n_idx=nidx, idx_stride=stride)
    ref, ref_lse = oracle.attention_rows(p, oracle.all_rows(p), nthreads=8)
    out, lse = run_int8_decode(w, q, kc, vc, ks, vsa[0], g, token_idx=idx, n_idx=nidx, split=256)
    assert np.abs(out - ref).max() <= 2e-3


def test_int8_128k_full_size():
    """4 x 8 KV heads x 131072 tokens x 128, 2 outlier channels x10 per head: bit-exact codes
    and scales over the whole cache, decode parity on sampled rows."""
    w = synth.workload("int8_128k")
    q, k, v, g = gen_kv(w)
    log_case("int8 128k full size")
    kc, ks = gpu_quant(k, g, 64)
    vc, vsa = gpu_quant(v, g, 0)
    ref_k, ref_ks = oracle.quant_partitions(g.B, g.KH, g.D, g.lens, g.seq_offset, g.stride_h, g.stride_t, k, 64, 2048)
    assert np.array_equal(ks, ref_ks)
    assert np.array_equal(kc, ref_k)
    del ref_k
    ref_v, ref_vs = oracle.quant_tensor(g.B, g.KH, g.D, g.lens, g.seq_offset, g.stride_h, g.stride_t, v)
    assert vsa[0] == np.float32(ref_vs)
    assert np.array_equal(vc, ref_v)
    del ref_v
    out, lse = run_int8_decode(w, q, kc, vc, ks, vsa[0], g, split=w.split_tokens)
    p = problem(w, q, kc, vc, g, k_scale=ks, k_part=64, k_scale_stride=2048, v_scale=float(vsa[0]))
    rng = np.random.default_rng(2)
    rows = [(int(b), int(h)) for b, h in zip(rng.integers(0, w.B, 12), rng.integers(0, w.QH, 12))] + [(3, 63)]
    ref, ref_lse = oracle.attention_rows(p, rows, nthreads=16)
    idx = [b * w.QH + h for b, h in rows]
    assert np.abs(out[idx] - ref).max() <= 2e-3
    assert np.abs(lse[idx] - ref_lse).max() <= 1e-3
    # informational: error of INT8 attention against the unquantised bf16 values (the page quotes ~0.4%)
    pb = problem(w, q, k, v, g)
    refb, _ = oracle.attention_rows(pb, rows[:4], nthreads=16)
    rel = np.linalg.norm(out[idx[:4]] - refb) / np.linalg.norm(refb)
    print(f"[info] int8 vs bf16 relative error on sampled rows: {rel:.4f}")
