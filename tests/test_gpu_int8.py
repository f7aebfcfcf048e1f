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
from gpu_helpers import DEV, dev_geom, host_threads, log_case, oracle_all_rows, problem, to_dev

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


@pytest.mark.parametrize("D,part,layout", [(64, 64, "head_major"), (256, 32, "token_major"), (40, 64, "head_major"),
                                           (128, 256, "token_major"), (64, 512, "head_major"), (128, 32, "head_major")])
def test_quant_geometries_bit_exact_and_nothing_written_outside_rows(D, part, layout):
    """Partition and per-tensor quantisation over head sizes with compile-time (64, 256) and run-time (40)
    row geometry and partitions from 32 to 512 tokens, ragged lengths: codes and scales bit-exact, and
    every code outside the sequences' valid rows left as the zeros it started from."""
    lens = np.array([1, 63, 64, 65, 700, 2049, 0, 130, 511, 513], np.int32)
    w = synth.workload("int8_128k", B=len(lens), KH=2, D=D, lens=lens, layout=layout, seed=60 + D + part)
    q, k, v, g = gen_kv(w)
    log_case(f"int8 quant geometry D={D} part={part} {layout}")
    mask = np.zeros(g.numel, bool)
    for b in range(g.B):
        for kh in range(g.KH):
            for t in range(lens[b]):
                o = g.seq_offset[b] + kh * g.stride_h + t * g.stride_t
                mask[o:o + g.D] = True
    stride = max(1, -(-int(lens.max()) // part))
    ref_codes, ref_scales = oracle.quant_partitions(g.B, g.KH, g.D, g.lens, g.seq_offset, g.stride_h, g.stride_t,
                                                    k, part, stride)
    codes, scales = gpu_quant(k, g, part)
    np.testing.assert_array_equal(codes[mask], ref_codes[mask])
    assert not codes[~mask].any()
    for b in range(g.B):
        for kh in range(g.KH):
            n = -(-int(lens[b]) // part)
            base = (b * g.KH + kh) * stride
            np.testing.assert_array_equal(scales[base:base + n], ref_scales[base:base + n])
    ref_v, ref_vs = oracle.quant_tensor(g.B, g.KH, g.D, g.lens, g.seq_offset, g.stride_h, g.stride_t, v)
    vc, vs = gpu_quant(v, g, 0)
    assert vs[0] == np.float32(ref_vs)
    np.testing.assert_array_equal(vc[mask], ref_v[mask])
    assert not vc[~mask].any()


def test_quant_rounds_exact_ties_to_even():
    """Values whose quotient by the scale is exactly a half-integer: max |x| = 254 gives scale 2, so
    x = 3, 5, -3, 1, 253 sit on ties (1.5, 2.5, -1.5, 0.5, 126.5) and round to even (2, 2, -2, 0, 126)."""
    lens = np.array([64], np.int32)
    w = synth.workload("int8_128k", B=1, KH=1, lens=lens, layout="head_major", seed=71)
    q, k, v, g = gen_kv(w)
    vals = np.array([254, 3, 5, -3, 1, 253, -253, 7, 0, 127, 129, -129], np.float32)
    kf = np.zeros(g.numel, np.float32)
    kf[:len(vals)] = vals
    k16 = (kf.view(np.uint32) >> 16).astype(np.uint16)       # all exactly representable in bf16
    codes, scales = gpu_quant(k16, g, 64)
    assert scales[0] == np.float32(2.0)
    expect = np.array([127, 2, 2, -2, 0, 126, -126, 4, 0, 64, 64, -64], np.int8)
    np.testing.assert_array_equal(codes[:len(vals)], expect)
    ref_codes, _ = oracle.quant_partitions(g.B, g.KH, g.D, g.lens, g.seq_offset, g.stride_h, g.stride_t, k16, 64, 1)
    np.testing.assert_array_equal(codes, ref_codes)


def test_quant_tiny_partitions_with_subnormal_scales():
    """Partitions whose max |x| is below 127 * 2^-126, so the scale is subnormal (and x / s still spans
    the code range): codes and scales bit-exact against the oracle's IEEE fp32 arithmetic."""
    lens = np.array([256], np.int32)
    w = synth.workload("int8_128k", B=1, KH=1, lens=lens, layout="head_major", seed=73)
    q, k, v, g = gen_kv(w)
    kf = (k.astype(np.uint32) << 16).view(np.float32).copy()
    for p_, mx in enumerate((1e-37, 3e-39, 1e-39, 4e-40)):   # one tiny magnitude per 64-token partition
        seg = slice(p_ * 64 * g.D, (p_ + 1) * 64 * g.D)
        kf[seg] = kf[seg] / np.abs(kf[seg]).max() * np.float32(mx)
    k16 = (kf.view(np.uint32) >> 16).astype(np.uint16)       # truncation keeps them tiny bf16 values
    ref_codes, ref_scales = oracle.quant_partitions(g.B, g.KH, g.D, g.lens, g.seq_offset, g.stride_h, g.stride_t,
                                                    k16, 64, 4)
    codes, scales = gpu_quant(k16, g, 64)
    assert (ref_scales < np.float32(2.0 ** -126)).all() and (ref_scales > 0).all()
    np.testing.assert_array_equal(scales, ref_scales)
    np.testing.assert_array_equal(codes, ref_codes)
    assert np.abs(codes.astype(np.int32)).max() == 127


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


def run_int8_decode(w, q, kc, vc, ks, vs, g, part=64, token_idx=None, n_idx=None, split=1024, **extra):
    qd = to_dev(q.reshape(-1)).view(w.B, w.QH, w.D)
    lse = torch.empty((w.B, w.QH), dtype=torch.float32, device=DEV)
    kw = dict(extra)
    if token_idx is not None:
        kw.update(token_idx=to_dev(token_idx), n_idx=to_dev(n_idx))
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


@pytest.mark.parametrize("G", [8, 24, 40])  # one 16-column block, one 32-column group, two groups
def test_int8_decode_with_kept_token_subset(G):
    lens = np.array([2000, 900], np.int32)
    w = synth.workload("int8_128k", B=2, KH=2, G=G, lens=lens, layout="token_major", seed=58)
    q, k, v, g = gen_kv(w)
    kc, ks = gpu_quant(k, g, 64)
    vc, vsa = gpu_quant(v, g, 0)
    rng = np.random.default_rng(5)
    stride = 600
    idx = np.zeros((4, stride), np.int32)
    nidx = np.array([600, 17, 300, 1], np.int32)
    for i in range(4):
        idx[i, :nidx[i]] = np.sort(rng.choice(lens[i // 2], size=nidx[i], replace=False))
    log_case(f"int8 decode kept subset G={G}")
    p = problem(w, q, kc, vc, g, k_scale=ks, k_part=64, k_scale_stride=-(-2000 // 64), v_scale=float(vsa[0]),
                tok_idx=idx.reshape(-1), n_idx=nidx, idx_stride=stride)
    ref, ref_lse = oracle.attention_rows(p, oracle.all_rows(p), nthreads=8)
    out, lse = run_int8_decode(w, q, kc, vc, ks, vsa[0], g, token_idx=idx, n_idx=nidx, split=256)
    assert np.abs(out - ref).max() <= 2e-3


def test_int8_128k_full_size():
    """4 x 8 KV heads x 131072 tokens x 128, 2 outlier channels x10 per head: bit-exact codes
    and scales over the whole cache, decode parity on every output row."""
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
    ref, ref_lse = oracle_all_rows(p)
    assert np.abs(out - ref).max() <= 2e-3
    assert np.abs(lse - ref_lse).max() <= 1e-3
    # informational: error of INT8 attention against the unquantised bf16 values (the page quotes ~0.4%)
    rows = [(0, 0), (1, 17), (2, 40), (3, 63)]
    pb = problem(w, q, k, v, g)
    refb, _ = oracle.attention_rows(pb, rows, nthreads=host_threads())
    idx = [b * w.QH + h for b, h in rows]
    rel = np.linalg.norm(out[idx] - refb) / np.linalg.norm(refb)
    print(f"[info] int8 vs bf16 relative error on four rows: {rel:.4f}")


# --- the page's INT8 schemes (§6 scheme table): query per row (A, B) or static per tensor (baseline);
# K per 64/128-token partition (A) or per tensor (B, baseline); V per tensor ---

SCHEMES = {
    "A64": dict(k_part=64, q_quant=pkg.QUANT_ROW),
    "A128": dict(k_part=128, q_quant=pkg.QUANT_ROW),
    "B": dict(k_part=0, q_quant=pkg.QUANT_ROW),
    "baseline": dict(k_part=0, q_quant=pkg.QUANT_STATIC),
}


def scheme_inputs(w, q, k, v, g, scheme, static_shrink=1.0):
    """GPU-quantised K/V codes for the scheme, plus the oracle's own int8 query (codes and per-row
    scales) and the oracle problem on those values."""
    sc = SCHEMES[scheme]
    kc, ks = gpu_quant(k, g, sc["k_part"])
    vc, vsa = gpu_quant(v, g, 0)
    rows = q.reshape(w.B * w.QH, w.D)
    q_scale = 0.0
    if sc["q_quant"] == pkg.QUANT_ROW:
        qc, qs = oracle.quant_rows(rows)
    else:
        # a static scale calibrated on this query (max|Q| / 127), optionally shrunk so that codes clamp
        q_scale = float(np.float32(np.abs(synth.bf16_bits_to_f32(rows)).max()) / np.float32(127.0)
                        * np.float32(static_shrink))
        qc = oracle.quant_static(rows, q_scale)
        qs = np.full(w.B * w.QH, q_scale, np.float32)
    if sc["k_part"]:
        stride = -(-int(g.max_len) // sc["k_part"])
        kk = dict(k_scale=ks, k_part=sc["k_part"], k_scale_stride=stride)
    else:
        kk = dict(k_scale=np.full(w.B * w.KH, ks[0], np.float32), k_part=1 << 30, k_scale_stride=1)
    p = problem(w, qc.reshape(q.shape), kc, vc, g, v_scale=float(vsa[0]), q_scale=qs, **kk)
    run = dict(part=sc["k_part"], q_quant=sc["q_quant"], q_scale=q_scale)
    return kc, vc, ks, vsa[0], p, run, qc, qs


@pytest.mark.parametrize("scheme", list(SCHEMES))
@pytest.mark.parametrize("G,D", [(8, 128), (4, 64)])
def test_int8_schemes_match_oracle(scheme, G, D):
    lens = np.array([3000, 1, 64, 1500, 0], np.int32)
    w = synth.workload("int8_128k", B=len(lens), KH=2, G=G, D=D, lens=lens, layout="token_major", seed=70 + G)
    q, k, v, g = gen_kv(w)
    log_case(f"int8 scheme {scheme} G={G} D={D}")
    kc, vc, ks, vs, p, run, _, _ = scheme_inputs(w, q, k, v, g, scheme)
    ref, ref_lse = oracle.attention_rows(p, oracle.all_rows(p), nthreads=8)
    fin = np.isfinite(ref_lse)
    for split in (1024, 0):
        log_case(f"int8 scheme {scheme} G={G} D={D} split={split}")
        out, lse = run_int8_decode(w, q, kc, vc, ks, vs, g, split=split, **run)
        assert np.abs(out - ref).max() <= 2e-3
        assert np.abs(lse[fin] - ref_lse[fin]).max() <= 1e-3
        assert np.all(np.isneginf(lse[~fin]))


def test_int8_static_query_scale_clamps():
    # a static scale below the query's range: the largest query values clamp to +-127 on both sides
    lens = np.array([900, 2100], np.int32)
    w = synth.workload("int8_128k", B=2, KH=2, G=8, lens=lens, layout="token_major", seed=77)
    q, k, v, g = gen_kv(w)
    log_case("int8 static query scale with clamping")
    kc, vc, ks, vs, p, run, qc, _ = scheme_inputs(w, q, k, v, g, "baseline", static_shrink=0.5)
    assert np.any(np.abs(qc) == 127) and np.count_nonzero(np.abs(qc) == 127) > 4
    ref, _ = oracle.attention_rows(p, oracle.all_rows(p), nthreads=8)
    out, _ = run_int8_decode(w, q, kc, vc, ks, vs, g, split=512, **run)
    assert np.abs(out - ref).max() <= 2e-3


@pytest.mark.parametrize("q_quant", [pkg.QUANT_ROW, pkg.QUANT_STATIC, pkg.QUANT_EXACT])
@pytest.mark.parametrize("D", [128, 64])
def test_query_codes_read_back_through_one_hot_keys(q_quant, D):
    """The kernel's query codes, bit for bit: with K row t = e_t (code 1, per-tensor scale 1),
    V row t = e_t and softmax scale 1, out[d] = exp(q_hat[d] - lse), so q_hat[d] = ln(out[d]) + lse
    and code[d] = q_hat[d] / s.  Each (b, qh) row has its own scale."""
    B, KH, G = 2, 2, 8
    geom = synth.dense_geometry(B, KH, D, D)
    kc = np.zeros((B, KH, D, D), np.int8)
    kc[:, :, np.arange(D), np.arange(D)] = 1
    q = synth.fill_q(78 + D, B, KH * G, D, synth.BF16).reshape(B * KH * G, D).copy()
    q[5] = 0                                       # an all-zero row: scale 0, codes 0
    qf = synth.bf16_bits_to_f32(q).astype(np.float64)
    static = float(np.float32(np.abs(qf).max()) / np.float32(127.0) * np.float32(0.75))
    log_case(f"query codes via one-hot keys q_quant={q_quant} D={D}")
    lse = torch.empty((B, KH * G), dtype=torch.float32, device=DEV)
    out, _ = pkg.attn_decode_splitkv(to_dev(q).view(B, KH * G, D), to_dev(kc.reshape(-1)), to_dev(kc.reshape(-1)),
                                     dev_geom(geom), G, lse=lse, k_scale=to_dev(np.ones(1, np.float32)),
                                     k_part_tokens=0, v_scale=1.0, softmax_scale=1.0, split_tokens=0,
                                     q_quant=q_quant, q_scale=static)
    torch.cuda.synchronize()
    out = out.cpu().numpy().reshape(B * KH * G, D).astype(np.float64)
    lse = lse.cpu().numpy().reshape(-1).astype(np.float64)
    qhat = np.log(out) + lse[:, None]
    if q_quant == pkg.QUANT_EXACT:
        # the 22-bit form reproduces the bf16 query to far below the read-back noise
        assert np.abs(qhat - qf).max() <= 1e-4
        return
    if q_quant == pkg.QUANT_ROW:
        codes, scales = oracle.quant_rows(q)
    else:
        codes = oracle.quant_static(q, static)
        scales = np.full(len(q), static, np.float32)
    live = scales > 0
    got = qhat[live] / scales[live, None].astype(np.float64)
    assert np.abs(got - np.rint(got)).max() <= 0.02
    np.testing.assert_array_equal(np.rint(got).astype(np.int32), codes[live].astype(np.int32))
    # the zero row: uniform softmax, q_hat = 0 (scale 0 per row; a static scale codes it as 0 too)
    assert np.abs(qhat[5]).max() <= 1e-5


def test_int8_scheme_a_128k_full_size():
    """Scheme A at full size (4 x 8 KV heads x 131072 tokens x 128, 64-token K partitions, per-row
    int8 query), in the benchmark's launch configuration, on every output row."""
    w = synth.workload("int8_128k")
    q, k, v, g = gen_kv(w)
    log_case("int8 scheme A 128k full size")
    kc, vc, ks, vs, p, run, _, _ = scheme_inputs(w, q, k, v, g, "A64")
    out, lse = run_int8_decode(w, q, kc, vc, ks, vs, g, split=w.split_tokens, **run)
    ref, ref_lse = oracle_all_rows(p)
    assert np.abs(out - ref).max() <= 2e-3
    assert np.abs(lse - ref_lse).max() <= 1e-3
