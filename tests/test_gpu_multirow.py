"""GPU parity of multi-row (speculative) decode: R query rows per sequence (the NVIDIA blog's
GEMM-M = (1 + draft) x G); row r attends to the first L - (R - 1) + r tokens.

Outputs against the fp64 oracle (2e-3, lse 1e-3, -inf for rows that see no token); and, as the
matrix-core columns are independent and the work split does not change, the last row of an R-row
step equals the one-row decode of that query bit for bit when both use one column block.
"""
import time

import numpy as np
import pytest
import torch

import long_context_decode_gqa_amd as pkg
import oracle
import synth
from gpu_helpers import DEV, dev_geom, host_threads, log_case, problem, to_dev

pytestmark = pytest.mark.gpu


def multirow_q(w, R, seed):
    q = synth.fill_q(seed, w.B, R * w.QH, w.D, synth.BF16)
    return np.ascontiguousarray(q.reshape(w.B, R, w.QH, w.D))


def run(w, q, k, v, g, R, **kw):
    qd = to_dev(q.reshape(-1)).view(w.B, R, w.QH, w.D) if R > 1 else to_dev(q.reshape(-1)).view(w.B, w.QH, w.D)
    lse = torch.empty((w.B, R, w.QH) if R > 1 else (w.B, w.QH), dtype=torch.float32, device=DEV)
    out, _ = pkg.attn_decode_splitkv(qd, k, v, dev_geom(g), w.G, lse=lse, q_rows=R, **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


# R * G columns per KV head: 16 or fewer (one 16-column block per wave), 17-32 (32-column waves),
# 33-64 (64-column waves over bf16, two 32-column groups over int8)
@pytest.mark.parametrize("R,G,D", [(2, 8, 128), (4, 4, 128), (2, 16, 64), (3, 8, 64), (8, 8, 128), (5, 8, 64),
                                   (8, 6, 128)])
@pytest.mark.parametrize("kv", ["bf16", "int8", "int8_qrow"])
def test_multirow_against_oracle(R, G, D, kv):
    lens = np.array([1, 2, 700, 4096, 0, 2049, 5], np.int32)
    w = synth.workload("gqa32k", B=len(lens), KH=2, G=G, D=D, lens=lens, layout="token_major", seed=140 + R + G)
    _, k, v, g = synth.generate(w)
    q = multirow_q(w, R, 141 + R)
    log_case(f"multirow R={R} G={G} D={D} {kv}")
    kw, pk = dict(split_tokens=0), {}
    if kv == "bf16":
        kd, vd, kh_, vh_ = to_dev(k), to_dev(v), k, v
    else:
        geom = dev_geom(g)
        kd, ks = pkg.kv_quant_int8(to_dev(k), geom, 64)
        vd, vs = pkg.kv_quant_int8(to_dev(v), geom, 0)
        torch.cuda.synchronize()
        kh_, vh_ = kd.cpu().numpy(), vd.cpu().numpy()
        kw.update(k_scale=ks, k_part_tokens=64, v_scale=float(vs.item()))
        pk = dict(k_scale=ks.cpu().numpy(), k_part=64, k_scale_stride=-(-int(g.max_len) // 64),
                  v_scale=float(vs.item()))
    qo = q
    if kv == "int8_qrow":
        kw["q_quant"] = pkg.QUANT_ROW
        qc, qs = oracle.quant_rows(q.reshape(-1, w.D))
        qo, pk["q_scale"] = qc.reshape(q.shape), qs
    out, lse = run(w, q, kd, vd, g, R, **kw)
    p = problem(w, np.ascontiguousarray(qo[:, 0]), kh_, vh_, g, **pk)
    p.q = qo
    rows = [(b, r, qh) for b in range(w.B) for r in range(R) for qh in range(w.QH)]
    ref, ref_lse = oracle.attention_multirow(p, R, rows, nthreads=8)
    out = out.reshape(-1, w.D)
    lse = lse.reshape(-1)
    assert np.abs(out - ref).max() <= 2e-3
    fin = np.isfinite(ref_lse)
    assert np.all(np.isneginf(lse[~fin]))
    assert np.abs(lse[fin] - ref_lse[fin]).max() <= 1e-3
    if R * G <= 16:
        # the last row sees the whole cache: the one-row decode of that query, bit for bit
        q1 = np.ascontiguousarray(q[:, R - 1])
        o1, l1 = run(w, q1, kd, vd, g, 1, **kw)
        np.testing.assert_array_equal(out.reshape(w.B, R, w.QH, w.D)[:, R - 1], o1)
        np.testing.assert_array_equal(lse.reshape(w.B, R, w.QH)[:, R - 1], l1)


def test_multirow_128k_full_size():
    """R = 2 at the 128K bf16 shape (4 x 8 KV heads x 131072, G = 8: the 16 matrix-core columns are
    full), in the benchmark's configuration: every row against the oracle, the last row bit-exact
    against the one-row decode."""
    w = synth.workload("dense128k")
    _, k, v, g = synth.generate(w)
    R = 2
    q = multirow_q(w, R, 150)
    log_case("multirow 128k full size")
    kd, vd = to_dev(k), to_dev(v)
    out, lse = run(w, q, kd, vd, g, R, split_tokens=w.split_tokens)
    o1, l1 = run(w, np.ascontiguousarray(q[:, 1]), kd, vd, g, 1, split_tokens=w.split_tokens)
    np.testing.assert_array_equal(out[:, 1], o1)
    np.testing.assert_array_equal(lse[:, 1], l1)
    p = problem(w, np.ascontiguousarray(q[:, 0]), k, v, g)
    p.q = q
    rows = [(b, r, qh) for b in range(w.B) for r in range(R) for qh in range(w.QH)]
    t0 = time.perf_counter()
    ref, ref_lse = oracle.attention_multirow(p, R, rows, nthreads=host_threads())
    print(f"[info] oracle over {len(rows)} rows: {time.perf_counter() - t0:.1f} s", flush=True)
    assert np.abs(out.reshape(-1, w.D) - ref).max() <= 2e-3
    assert np.abs(lse.reshape(-1) - ref_lse).max() <= 1e-3


def test_multirow_128k_eight_rows():
    """R = 8 at the 128K bf16 shape (64 columns per KV head: 64-column waves over a full grid with
    non-temporal loads, the benchmark's launch): every row against the oracle."""
    w = synth.workload("dense128k")
    _, k, v, g = synth.generate(w)
    R = 8
    q = multirow_q(w, R, 152)
    log_case("multirow 128k eight rows")
    out, lse = run(w, q, to_dev(k), to_dev(v), g, R, split_tokens=w.split_tokens)
    p = problem(w, np.ascontiguousarray(q[:, 0]), k, v, g)
    p.q = q
    rows = [(b, r, qh) for b in range(w.B) for r in range(R) for qh in range(w.QH)]
    t0 = time.perf_counter()
    ref, ref_lse = oracle.attention_multirow(p, R, rows, nthreads=host_threads())
    print(f"[info] oracle over {len(rows)} rows: {time.perf_counter() - t0:.1f} s", flush=True)
    assert np.abs(out.reshape(-1, w.D) - ref).max() <= 2e-3
    assert np.abs(lse.reshape(-1) - ref_lse).max() <= 1e-3


@pytest.mark.parametrize("D", [128, 64])
def test_multirow_paged_full_grid(D):
    """R = 8 over a head-major paged pool with enough tiles for the full-grid launch (64-column
    waves, page table, non-temporal loads): bit for bit the contiguous decode, and against the
    oracle."""
    from test_gpu_paged import make_pool, paged_geom
    L, P = 40960 * 128 // D, 64
    w = synth.workload("dense128k", L=L, D=D)
    _, k, v, g = synth.generate(w)
    R = 8
    q = multirow_q(w, R, 153)
    log_case("multirow paged full grid")
    kw = dict(split_tokens=w.split_tokens)
    out_c, lse_c = run(w, q, to_dev(k), to_dev(v), g, R, **kw)
    kp, table, st, sh, ps = make_pool(k, g, P, "head_major", 17, np.uint16(0x7FC0))
    vp, _, _, _, _ = make_pool(v, g, P, "head_major", 17, np.uint16(0x7FC0))
    qd = to_dev(q.reshape(-1)).view(w.B, R, w.QH, w.D)
    lse_p = torch.empty((w.B, R, w.QH), dtype=torch.float32, device=DEV)
    out_p, _ = pkg.attn_decode_splitkv(qd, to_dev(kp), to_dev(vp), paged_geom(g, table, P, st, sh, ps), w.G,
                                       lse=lse_p, q_rows=R, **kw)
    torch.cuda.synchronize()
    out_p, lse_p = out_p.float().cpu().numpy(), lse_p.cpu().numpy()
    assert np.isfinite(out_p).all()
    np.testing.assert_array_equal(out_p, out_c)
    np.testing.assert_array_equal(lse_p, lse_c)
    p = problem(w, np.ascontiguousarray(q[:, 0]), k, v, g)
    p.q = q
    rows = [(b, r, qh) for b in range(w.B) for r in range(R) for qh in range(w.QH)]
    ref, ref_lse = oracle.attention_multirow(p, R, rows, nthreads=host_threads())
    assert np.abs(out_c.reshape(-1, w.D) - ref).max() <= 2e-3
    assert np.abs(lse_c.reshape(-1) - ref_lse).max() <= 1e-3


@pytest.mark.parametrize("D", [128, 64])
def test_multirow_four_rows_full_grid(D):
    """R = 4 (32-column waves, one column group) with enough tiles for the full-grid launch
    (non-temporal loads), contiguous and over a head-major paged pool: bit for bit the same, and
    against the oracle."""
    from test_gpu_paged import make_pool, paged_geom
    L, P = 40960 * 128 // D, 64
    w = synth.workload("dense128k", L=L, D=D)
    _, k, v, g = synth.generate(w)
    R = 4
    q = multirow_q(w, R, 154)
    log_case("multirow four rows full grid")
    kw = dict(split_tokens=w.split_tokens)
    out_c, lse_c = run(w, q, to_dev(k), to_dev(v), g, R, **kw)
    kp, table, st, sh, ps = make_pool(k, g, P, "head_major", 19, np.uint16(0x7FC0))
    vp, _, _, _, _ = make_pool(v, g, P, "head_major", 19, np.uint16(0x7FC0))
    qd = to_dev(q.reshape(-1)).view(w.B, R, w.QH, w.D)
    lse_p = torch.empty((w.B, R, w.QH), dtype=torch.float32, device=DEV)
    out_p, _ = pkg.attn_decode_splitkv(qd, to_dev(kp), to_dev(vp), paged_geom(g, table, P, st, sh, ps), w.G,
                                       lse=lse_p, q_rows=R, **kw)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out_p.float().cpu().numpy(), out_c)
    np.testing.assert_array_equal(lse_p.cpu().numpy(), lse_c)
    p = problem(w, np.ascontiguousarray(q[:, 0]), k, v, g)
    p.q = q
    rows = [(b, r, qh) for b in range(w.B) for r in range(R) for qh in range(w.QH)]
    ref, ref_lse = oracle.attention_multirow(p, R, rows, nthreads=host_threads())
    assert np.abs(out_c.reshape(-1, w.D) - ref).max() <= 2e-3
    assert np.abs(lse_c.reshape(-1) - ref_lse).max() <= 1e-3
