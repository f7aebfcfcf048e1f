"""GPU parity of decode over a paged KV cache ("注意力优化" 结构 4, PagedAttention).

The same logical cache is laid out contiguously and in a page pool with scrambled page
order (token-major or head-major pages, NaN or random values in the unused rows of the last
pages).  With the caller's split_tokens the work split depends only on the lengths, so the paged
decode must reproduce the contiguous decode bit for bit; it is also compared with the fp64 oracle
on the logical values.  (The library's default split runs more, shorter ranges over token-major
pages, so there the comparison is to the oracle and within tolerance.)
"""
import math

import numpy as np
import pytest
import torch

import long_context_decode_gqa_amd as pkg
import oracle
import synth
from gpu_helpers import DEV, dev_geom, log_case, oracle_all_rows, problem, to_dev

pytestmark = pytest.mark.gpu


def logical_rows(x, g, b, kh, L):
    off = g.seq_offset[b] + kh * g.stride_h
    return x[off + np.arange(L)[:, None] * g.stride_t + np.arange(g.D)[None, :]]


def make_pool(x, g, P, layout, seed, junk):
    """Page pool holding the logical rows of x (geometry g), its block table and strides."""
    rng = np.random.default_rng(seed)
    B, KH, D = g.B, g.KH, g.D
    lens = [int(L) for L in g.lens]
    need = [-(-L // P) for L in lens]
    total = sum(need) + 3
    perm = rng.permutation(total)
    pool = np.full((total, P, KH, D) if layout == "token_major" else (total, KH, P, D), junk, dtype=x.dtype)
    if x.dtype == np.int8:
        pool[...] = rng.integers(-127, 128, size=pool.shape).astype(np.int8)
    table = np.zeros((B, max(1, -(-int(g.max_len) // P))), np.int32)
    table[...] = perm[-1]  # entries past a sequence's pages name a spare page
    nxt = 0
    for b in range(B):
        if need[b] == 0:
            continue
        pages = perm[nxt:nxt + need[b]]
        nxt += need[b]
        table[b, :need[b]] = pages
        for kh in range(KH):
            rows = logical_rows(x, g, b, kh, lens[b])
            full = (lens[b] // P) * P
            if layout == "token_major":
                pool[pages[:full // P], :, kh] = rows[:full].reshape(-1, P, D)
                if full < lens[b]:
                    pool[pages[-1], :lens[b] - full, kh] = rows[full:]
            else:
                pool[pages[:full // P], kh] = rows[:full].reshape(-1, P, D)
                if full < lens[b]:
                    pool[pages[-1], kh, :lens[b] - full] = rows[full:]
    if layout == "token_major":
        st, sh, ps = KH * D, D, P * KH * D
    else:
        st, sh, ps = D, P * D, KH * P * D
    return pool.reshape(-1), table, st, sh, ps


def paged_geom(g, table, P, st, sh, ps):
    return pkg.KVGeometry(g.B, g.KH, g.D, int(g.max_len), torch.from_numpy(g.lens).to(DEV), None, sh, st,
                          block_table=torch.from_numpy(table).to(DEV), page_tokens=P, page_stride=ps)


def run(qd, k, v, geom, G, B, QH, **kw):
    lse = torch.empty((B, QH), dtype=torch.float32, device=DEV)
    out, _ = pkg.attn_decode_splitkv(qd, k, v, geom, G, lse=lse, **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("P,layout", [(32, "token_major"), (64, "head_major"), (256, "token_major")])
@pytest.mark.parametrize("kv", ["bf16", "int8", "int8_qrow"])
@pytest.mark.parametrize("D", [128, 64])
def test_paged_equals_contiguous_bit_exact(P, layout, kv, D):
    lens = np.array([1, 700, 4096, 2049, 0, 33], np.int32)
    # the contiguous cache in the pool's row order (any order gives the same bits)
    w = synth.workload("gqa32k", B=len(lens), KH=2, G=8, D=D, lens=lens, layout=layout, seed=130 + P)
    q, k, v, g = synth.generate(w)
    log_case(f"paged P={P} {layout} {kv} D={D}")
    qd = to_dev(q.reshape(-1)).view(w.B, w.QH, w.D)
    kw = dict(split_tokens=4096)
    if kv == "bf16":
        kx, vx = k, v
        junk = np.uint16(0x7FC0)  # NaN: rows past L must never be read
    else:
        geom_c = dev_geom(g)
        kc, ks = pkg.kv_quant_int8(to_dev(k), geom_c, 64)
        vc, vs = pkg.kv_quant_int8(to_dev(v), geom_c, 0)
        torch.cuda.synchronize()
        kx, vx = kc.cpu().numpy(), vc.cpu().numpy()
        junk = np.int8(0)
        kw.update(k_scale=ks, k_part_tokens=64, v_scale=float(vs.item()))
        if kv == "int8_qrow":
            kw["q_quant"] = pkg.QUANT_ROW
    out_c, lse_c = run(qd, to_dev(kx), to_dev(vx), dev_geom(g), w.G, w.B, w.QH, **kw)
    kp, table, st, sh, ps = make_pool(kx, g, P, layout, 7 + P, junk)
    vp, _, _, _, _ = make_pool(vx, g, P, layout, 7 + P, junk)
    out_p, lse_p = run(qd, to_dev(kp), to_dev(vp), paged_geom(g, table, P, st, sh, ps), w.G, w.B, w.QH, **kw)
    assert np.isfinite(out_p).all()
    np.testing.assert_array_equal(out_p, out_c)
    np.testing.assert_array_equal(lse_p, lse_c)
    if kv == "bf16":
        p = problem(w, q, k, v, g)
        ref, _ = oracle.attention_rows(p, oracle.all_rows(p), nthreads=8)
        assert np.abs(out_p.reshape(-1, w.D) - ref).max() <= 2e-3


@pytest.mark.parametrize("P,layout", [(64, "head_major"), (32, "token_major")])
@pytest.mark.parametrize("D", [128, 64])
def test_paged_64_column_waves_equal_contiguous(P, layout, D):
    # 48 query heads per KV head over a bf16 cache: 64-column waves (four
    # 16-column blocks per wave), contiguous and paged, bit for bit, and
    # against the oracle
    lens = np.array([3000, 1, 4097, 0, 640], np.int32)
    w = synth.workload("gqa32k", B=len(lens), KH=2, G=48, D=D, lens=lens, layout=layout, seed=150 + P + D)
    q, k, v, g = synth.generate(w)
    log_case(f"64-column waves P={P} {layout} D={D}")
    qd = to_dev(q.reshape(-1)).view(w.B, w.QH, w.D)
    kw = dict(split_tokens=1024)
    out_c, lse_c = run(qd, to_dev(k), to_dev(v), dev_geom(g), w.G, w.B, w.QH, **kw)
    junk = np.uint16(0x7FC0)  # NaN: rows past L must never be read
    kp, table, st, sh, ps = make_pool(k, g, P, layout, 9 + P, junk)
    vp, _, _, _, _ = make_pool(v, g, P, layout, 9 + P, junk)
    out_p, lse_p = run(qd, to_dev(kp), to_dev(vp), paged_geom(g, table, P, st, sh, ps), w.G, w.B, w.QH, **kw)
    assert np.isfinite(out_p).all()
    np.testing.assert_array_equal(out_p, out_c)
    np.testing.assert_array_equal(lse_p, lse_c)
    p = problem(w, q, k, v, g)
    ref, ref_lse = oracle.attention_rows(p, oracle.all_rows(p), nthreads=8)
    assert np.abs(out_c.reshape(-1, w.D) - ref).max() <= 2e-3
    live = np.isfinite(ref_lse)
    assert np.abs(lse_c.reshape(-1)[live] - ref_lse[live]).max() <= 1e-3


def test_paged_128k_full_size_equals_contiguous():
    """The 128K bf16 workload (4 x 8 KV heads x 131072 tokens) in scrambled pools of 64-token
    pages.  In the benchmark's launch configuration (the library's default split) head-major
    pages and the same data packed token-major are bit-identical to the dense cache, and token-major
    pages, whose default split differs, match every row of the oracle and the dense result within
    tolerance; with the same split_tokens as the dense cache's default (4096) token-major pages are
    bit-identical too."""
    w = synth.workload("dense128k")
    q, k, v, g = synth.generate(w)
    log_case("paged 128k full size")
    qd = to_dev(q.reshape(-1)).view(w.B, w.QH, w.D)
    P = 64
    out_c, lse_c = run(qd, to_dev(k), to_dev(v), dev_geom(g), w.G, w.B, w.QH, split_tokens=w.split_tokens)
    kp, table, st, sh, ps = make_pool(k, g, P, "head_major", 11, np.uint16(0x7FC0))
    vp, _, _, _, _ = make_pool(v, g, P, "head_major", 11, np.uint16(0x7FC0))
    out_p, lse_p = run(qd, to_dev(kp), to_dev(vp), paged_geom(g, table, P, st, sh, ps), w.G, w.B, w.QH,
                       split_tokens=w.split_tokens)
    del kp, vp
    np.testing.assert_array_equal(out_p, out_c)
    np.testing.assert_array_equal(lse_p, lse_c)
    # token-major: the same cache packed [B*L][KH][D], and in token-major pages
    L = int(w.lens[0])
    wt = synth.workload("dense128k", layout="token_major")
    gt = wt.geometry()
    kt = np.ascontiguousarray(k.reshape(w.B, w.KH, L, w.D).transpose(0, 2, 1, 3)).reshape(-1)
    vt = np.ascontiguousarray(v.reshape(w.B, w.KH, L, w.D).transpose(0, 2, 1, 3)).reshape(-1)
    out_t, lse_t = run(qd, to_dev(kt), to_dev(vt), dev_geom(gt), w.G, w.B, w.QH, split_tokens=w.split_tokens)
    kp, table, st, sh, ps = make_pool(k, g, P, "token_major", 11, np.uint16(0x7FC0))
    vp, _, _, _, _ = make_pool(v, g, P, "token_major", 11, np.uint16(0x7FC0))
    kpd, vpd, pg = to_dev(kp), to_dev(vp), paged_geom(g, table, P, st, sh, ps)
    del kp, vp, kt, vt
    out_p, lse_p = run(qd, kpd, vpd, pg, w.G, w.B, w.QH, split_tokens=w.split_tokens)
    out_s, lse_s = run(qd, kpd, vpd, pg, w.G, w.B, w.QH, split_tokens=4096)
    np.testing.assert_array_equal(out_t, out_c)
    np.testing.assert_array_equal(lse_t, lse_c)
    np.testing.assert_array_equal(out_s, out_c)
    np.testing.assert_array_equal(lse_s, lse_c)
    assert np.abs(out_p - out_c).max() <= 1e-5
    assert np.abs(lse_p - lse_c).max() <= 1e-5
    ref, ref_lse = oracle_all_rows(problem(w, q, k, v, g))
    assert np.abs(out_p.reshape(-1, w.D) - ref).max() <= 2e-3
    assert np.abs(lse_p.reshape(-1) - ref_lse).max() <= 1e-3


# --- the rest of the path over a paged cache: quantisation when rows are written, the cached
# value norms, and OAM selection read the pool through the same block table; each must equal
# its contiguous counterpart bit for bit (the contiguous results are compared with the oracle
# in test_gpu_int8.py and test_gpu_oam.py) ---

def pool_rows(pool, g, table, P, st, sh, ps, b, kh, L):
    """The logical rows (b, kh, 0..L-1) of a page pool, as an array [L, D]."""
    t = np.arange(L)
    start = table[b, t // P].astype(np.int64) * ps + kh * sh + (t % P) * st
    return pool[start[:, None] + np.arange(g.D)[None, :]]


def valid_mask(g, table, P, st, sh, ps, n):
    m = np.zeros(n, bool)
    for b in range(g.B):
        for kh in range(g.KH):
            L = int(g.lens[b])
            t = np.arange(L)
            start = table[b, t // P].astype(np.int64) * ps + kh * sh + (t % P) * st
            m[(start[:, None] + np.arange(g.D)[None, :]).reshape(-1)] = True
    return m


@pytest.mark.parametrize("P,layout,part", [(32, "token_major", 64), (64, "head_major", 64), (128, "token_major", 16),
                                           (64, "head_major", 128)])
def test_paged_quantisation_equals_contiguous(P, layout, part):
    """K per token partition (partitions may straddle pages) and V per tensor over a page pool:
    codes of every logical row and the scales equal the contiguous quantiser's; pool rows that
    hold no token keep the zeros the codes started from."""
    lens = np.array([1, 63, 700, 2049, 0, 130], np.int32)
    w = synth.workload("int8_128k", B=len(lens), KH=2, lens=lens, layout="head_major", seed=200 + P + part)
    q, k, v, g = synth.generate(w)
    log_case(f"paged quant P={P} {layout} part={part}")
    geom = dev_geom(g)
    kc, ks = pkg.kv_quant_int8(to_dev(k), geom, part)
    vc, vs = pkg.kv_quant_int8(to_dev(v), geom, 0)
    kp, table, st, sh, ps = make_pool(k, g, P, layout, seed=P, junk=0)
    vp, _, _, _, _ = make_pool(v, g, P, layout, seed=P, junk=0)
    pg = paged_geom(g, table, P, st, sh, ps)
    kcp, ksp = pkg.kv_quant_int8(to_dev(kp), pg, part)
    vcp, vsp = pkg.kv_quant_int8(to_dev(vp), pg, 0)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ksp.cpu().numpy(), ks.cpu().numpy())
    assert vsp.item() == vs.item()
    kc, vc, kcp, vcp = kc.cpu().numpy(), vc.cpu().numpy(), kcp.cpu().numpy(), vcp.cpu().numpy()
    for b in range(g.B):
        for kh in range(g.KH):
            L = int(lens[b])
            np.testing.assert_array_equal(pool_rows(kcp, g, table, P, st, sh, ps, b, kh, L),
                                          logical_rows(kc, g, b, kh, L))
            np.testing.assert_array_equal(pool_rows(vcp, g, table, P, st, sh, ps, b, kh, L),
                                          logical_rows(vc, g, b, kh, L))
    m = valid_mask(g, table, P, st, sh, ps, kcp.size)
    assert not kcp[~m].any() and not vcp[~m].any()


@pytest.mark.parametrize("P,layout,kv", [(32, "token_major", "bf16"), (64, "head_major", "bf16"),
                                         (64, "token_major", "int8")])
def test_paged_value_norms_and_oam_equal_contiguous(P, layout, kv):
    """Value log-norms, OAM scores and kept sets (token and 64-token block selection, value term
    cached or read from V) over a page pool equal the contiguous results bit for bit."""
    lens = np.array([9000, 1, 8192, 3000, 0, 16500], np.int32)
    w = synth.workload("oam_128k", B=len(lens), KH=2, lens=lens, layout="head_major", seed=300 + P)
    q, k, v, g = synth.generate(w)
    log_case(f"paged oam P={P} {layout} {kv}")
    geom = dev_geom(g)
    qd = to_dev(q.reshape(-1)).view(w.B, w.QH, w.D)
    kd, vd = to_dev(k), to_dev(v)
    extra, vsc = {}, 1.0
    if kv == "int8":
        kd, ks = pkg.kv_quant_int8(kd, geom, 64)
        vd, vs = pkg.kv_quant_int8(vd, geom, 0)
        torch.cuda.synchronize()
        vsc = float(vs.item())
        extra = dict(k_scale=ks, k_part_tokens=64, v_scale=vsc)
    kh_, vh_ = (kd.cpu().numpy(), vd.cpu().numpy()) if kv == "int8" else (k, v)   # host bf16 stays uint16
    kp, table, st, sh, ps = make_pool(kh_, g, P, layout, seed=P + 1, junk=0)
    vp, _, _, _, _ = make_pool(vh_, g, P, layout, seed=P + 1, junk=0)
    pg = paged_geom(g, table, P, st, sh, ps)
    kpd, vpd = to_dev(kp), to_dev(vp)
    vl = pkg.oam_value_lognorm(vd, geom, w.eps, v_scale=vsc)
    vlp = pkg.oam_value_lognorm(vpd, pg, w.eps, v_scale=vsc)
    torch.cuda.synchronize()
    vl_h, vlp_h = vl.cpu().numpy(), vlp.cpu().numpy()
    for b in range(g.B):
        for kh in range(g.KH):
            L = int(lens[b])
            np.testing.assert_array_equal(vlp_h[b * g.KH + kh, :L], vl_h[b * g.KH + kh, :L])
    for mode in (dict(vlog=vl), dict(v=vd), dict(vlog=vl, block_tokens=64)):
        top_k = 8 if "block_tokens" in mode else 700
        n = w.B * w.KH
        sc = torch.full((n, int(g.max_len)), float("nan"), dtype=torch.float32, device=DEV)
        scp = torch.full_like(sc, float("nan"))
        modep = {kk: (vpd if kk == "v" else vv) for kk, vv in mode.items()}
        idx, nk = pkg.oam_score_topk(qd, kd, geom, w.G, top_k, scores_out=sc, beta=w.beta, eps=w.eps, **mode, **extra)
        idxp, nkp = pkg.oam_score_topk(qd, kpd, pg, w.G, top_k, scores_out=scp, beta=w.beta, eps=w.eps, **modep,
                                       **extra)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(nkp.cpu().numpy(), nk.cpu().numpy())
        np.testing.assert_array_equal(idxp.cpu().numpy(), idx.cpu().numpy())
        s_h, sp_h = sc.cpu().numpy(), scp.cpu().numpy()
        for b in range(g.B):
            for kh in range(g.KH):
                L = int(lens[b])
                np.testing.assert_array_equal(sp_h[b * g.KH + kh, :L], s_h[b * g.KH + kh, :L])


@pytest.mark.parametrize("kv", ["bf16", "int8", "int8_qrow"])
@pytest.mark.parametrize("D", [128, 64])
def test_paged_full_grid_equals_contiguous(kv, D):
    """Caches with enough tiles for the full-grid launch (non-temporal loads), contiguous and in
    head-major pages: bit for bit the same, and against the oracle on the cached values."""
    L, P = 40960 * 128 // D, 64
    w = synth.workload("dense128k", L=L, D=D)
    q, k, v, g = synth.generate(w)
    log_case(f"paged full grid {kv} D={D}")
    qd = to_dev(q.reshape(-1)).view(w.B, w.QH, w.D)
    geom_c = dev_geom(g)
    kw, pk, qo = dict(split_tokens=w.split_tokens), {}, q
    if kv == "bf16":
        kx, vx, junk = k, v, np.uint16(0x7FC0)
    else:
        kc, ks = pkg.kv_quant_int8(to_dev(k), geom_c, 64)
        vc, vs = pkg.kv_quant_int8(to_dev(v), geom_c, 0)
        torch.cuda.synchronize()
        kx, vx, junk = kc.cpu().numpy(), vc.cpu().numpy(), np.int8(0)
        del kc, vc
        kw.update(k_scale=ks, k_part_tokens=64, v_scale=float(vs.item()))
        pk = dict(k_scale=ks.cpu().numpy(), k_part=64, k_scale_stride=-(-L // 64), v_scale=float(vs.item()))
        if kv == "int8_qrow":
            kw["q_quant"] = pkg.QUANT_ROW
            qc, qs = oracle.quant_rows(q.reshape(-1, w.D))
            qo, pk["q_scale"] = qc.reshape(q.shape), qs
    out_c, lse_c = run(qd, to_dev(kx), to_dev(vx), geom_c, w.G, w.B, w.QH, **kw)
    kp, table, st, sh, ps = make_pool(kx, g, P, "head_major", 23, junk)
    vp, _, _, _, _ = make_pool(vx, g, P, "head_major", 23, junk)
    out_p, lse_p = run(qd, to_dev(kp), to_dev(vp), paged_geom(g, table, P, st, sh, ps), w.G, w.B, w.QH, **kw)
    np.testing.assert_array_equal(out_p, out_c)
    np.testing.assert_array_equal(lse_p, lse_c)
    p = problem(w, qo, kx, vx, g, **pk)
    ref, ref_lse = oracle_all_rows(p)
    assert np.abs(out_c.reshape(-1, w.D) - ref).max() <= 2e-3
    assert np.abs(lse_c.reshape(-1) - ref_lse).max() <= 1e-3
