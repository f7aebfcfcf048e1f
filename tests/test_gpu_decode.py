"""GPU parity of attn_decode_splitkv / attn_merge_lse against the fp64 oracle.

Tolerance: max |gpu - oracle| <= 2e-3 on fp32 outputs (fp32 accumulation);
bf16 outputs additionally allow half a bf16 ulp of the value.  lse within
1e-3.  Bitwise repeatability: no floating-point atomics anywhere.
"""
import math

import numpy as np
import pytest
import torch

import long_context_decode_gqa_amd as pkg
import oracle
import synth
from gpu_helpers import DEV, bf16_to_f32, dev_geom, log_case, oracle_all_rows, problem, to_dev

pytestmark = pytest.mark.gpu
TOL = 2e-3


def run_decode(w, q, k, v, g, out_dtype=torch.float32, **kw):
    qd = to_dev(q.reshape(-1)).view(w.B, w.QH, w.D)
    kd, vd = to_dev(k), to_dev(v)
    lse = torch.full((w.B, w.QH), 7.0, dtype=torch.float32, device=DEV)
    out, _ = pkg.attn_decode_splitkv(qd, kd, vd, dev_geom(g), w.G, lse=lse, out_dtype=out_dtype, **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().reshape(w.B * w.QH, w.D), lse.cpu().numpy().reshape(-1)


def check(out, lse, ref, ref_lse, bf16_out=False, tol=TOL):
    tol_arr = tol + (np.abs(ref) * 2.0 ** -9 if bf16_out else 0.0)
    err = np.abs(out - ref)
    assert np.all(err <= tol_arr), f"max err {err.max():.3e}"
    fin = np.isfinite(ref_lse)
    assert np.all(np.isneginf(lse[~fin])), "empty rows must have lse = -inf"
    assert np.all(np.abs(lse[fin] - ref_lse[fin]) <= 1e-3), f"lse err {np.abs(lse[fin]-ref_lse[fin]).max():.3e}"


@pytest.mark.parametrize("split", [0, 1024, 256, 64])
def test_tiny_fp32_unsplit_and_split(split):
    w = synth.workload("tiny")
    q, k, v, g = synth.generate(w)
    log_case(f"tiny fp32 split={split}")
    out, lse = run_decode(w, q, k, v, g, split_tokens=split)
    p = problem(w, q, k, v, g)
    ref, ref_lse = oracle.attention_rows(p, oracle.all_rows(p))
    check(out, lse, ref, ref_lse, tol=1e-5)


# split 4096 / 16384: one worker and one chunk per lane, so the decode writes the rows itself
# (empty lanes included) and no merge runs
@pytest.mark.parametrize("D,G,split", [(4, 3, 0), (36, 20, 64), (100, 7, 96), (256, 16, 0), (64, 33, 256),
                                       (100, 7, 4096), (64, 33, 16384)])
def test_fp32_ragged_head_sizes_and_groups(D, G, split):
    """The fp32 path over ragged lengths (empty, shorter than a tile, tile and chunk boundaries)
    for head sizes 4..256 and group sizes beyond one 16-head block."""
    lens = np.array([0, 1, 31, 32, 33, 300, 1000], np.int32)
    w = synth.workload("tiny", B=len(lens), KH=2, G=G, D=D, lens=lens, layout="token_major", seed=120 + D)
    q, k, v, g = synth.generate(w)
    log_case(f"fp32 ragged D={D} G={G} split={split}")
    out, lse = run_decode(w, q, k, v, g, split_tokens=split)
    p = problem(w, q, k, v, g)
    ref, ref_lse = oracle.attention_rows(p, oracle.all_rows(p))
    check(out, lse, ref, ref_lse, tol=1e-5)


@pytest.mark.parametrize("split", [64, 4096])
def test_fp32_kept_token_subset(split):
    """The fp32 path with a per-(sequence, KV head) list of kept positions (split 4096: one worker,
    no merge)."""
    lens = np.array([500, 77, 0, 1200], np.int32)
    w = synth.workload("tiny", B=len(lens), KH=2, G=4, D=64, lens=lens, layout="head_major", seed=131)
    q, k, v, g = synth.generate(w)
    rng = np.random.default_rng(5)
    stride = 256
    idx = np.full((w.B, w.KH, stride), -1, np.int32)
    nidx = np.zeros((w.B, w.KH), np.int32)
    for b in range(w.B):
        for kh in range(w.KH):
            n = min(int(lens[b]), int(rng.integers(1, stride + 1)))
            idx[b, kh, :n] = np.sort(rng.choice(int(lens[b]), n, replace=False)) if n else []
            nidx[b, kh] = n
    log_case(f"fp32 kept tokens split={split}")
    out, lse = run_decode(w, q, k, v, g, split_tokens=split, token_idx=to_dev(idx), n_idx=to_dev(nidx))
    p = problem(w, q, k, v, g, tok_idx=idx.reshape(-1), n_idx=nidx.reshape(-1), idx_stride=stride)
    ref, ref_lse = oracle.attention_rows(p, oracle.all_rows(p))
    check(out, lse, ref, ref_lse, tol=1e-5)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 4, 8, 16, 24])
def test_bf16_ragged_tails_and_group_sizes(D, G):
    lens = np.array([1, 63, 64, 65, 1023, 1025, 2500, 0], np.int32)
    w = synth.workload("gqa32k", B=len(lens), G=G, D=D, KH=2, lens=lens, layout="token_major", seed=100 + G)
    q, k, v, g = synth.generate(w)
    log_case(f"bf16 ragged D={D} G={G}")
    p = problem(w, q, k, v, g)
    ref, ref_lse = oracle.attention_rows(p, oracle.all_rows(p), nthreads=8)
    # split 0: the library's default chunk size
    for split, od in ((1024, torch.float32), (256, torch.bfloat16), (0, torch.float32), (0, torch.bfloat16)):
        log_case(f"bf16 ragged D={D} G={G} split={split} out={od}")
        out, lse = run_decode(w, q, k, v, g, out_dtype=od, split_tokens=split)
        check(out, lse, ref, ref_lse, bf16_out=(od == torch.bfloat16))


def test_bf16_head_major_layout_and_lse():
    lens = np.array([4000, 700, 33], np.int32)
    w = synth.workload("gqa32k", B=3, KH=4, G=8, lens=lens, layout="head_major", seed=7)
    q, k, v, g = synth.generate(w)
    log_case("bf16 head-major")
    p = problem(w, q, k, v, g)
    ref, ref_lse = oracle.attention_rows(p, oracle.all_rows(p), nthreads=8)
    for split in (512, 0):
        out, lse = run_decode(w, q, k, v, g, split_tokens=split)
        check(out, lse, ref, ref_lse)


def test_bitwise_repeatable():
    w = synth.workload("gqa32k", B=3, L=5000, seed=9)
    q, k, v, g = synth.generate(w)
    log_case("repeatability")
    a = run_decode(w, q, k, v, g, split_tokens=512)
    b = run_decode(w, q, k, v, g, split_tokens=512)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_large_scores_and_peaked_softmax():
    # scaled-up q makes the softmax nearly one-hot; probabilities near 1 must not lose accuracy
    w = synth.workload("gqa32k", B=2, L=3000, seed=10)
    q, k, v, g = synth.generate(w)
    qf = synth.bf16_bits_to_f32(q) * np.float32(6.0)
    q6 = ((qf.view(np.uint32) + 0x7FFF + ((qf.view(np.uint32) >> 16) & 1)) >> 16).astype(np.uint16)
    log_case("peaked softmax")
    p = problem(w, q6, k, v, g)
    ref, ref_lse = oracle.attention_rows(p, oracle.all_rows(p), nthreads=8)
    out, lse = run_decode(w, q6, k, v, g, split_tokens=1024)
    check(out, lse, ref, ref_lse)


@pytest.mark.parametrize("G", [8, 24, 48])  # one 16-column block, one 32-column group, two groups
def test_token_index_subset(G):
    lens = np.array([3000, 1500], np.int32)
    w = synth.workload("gqa32k", B=2, KH=2, G=G, lens=lens, layout="token_major", seed=11)
    q, k, v, g = synth.generate(w)
    rng = np.random.default_rng(0)
    stride = 700
    lists = []
    for b in range(w.B):
        for kh in range(w.KH):
            n = [700, 1, 333, 0][b * 2 + kh]
            lists.append(np.sort(rng.choice(lens[b], size=n, replace=False)).astype(np.int32))
    idx = np.zeros((w.B * w.KH, stride), np.int32)
    nidx = np.array([len(x) for x in lists], np.int32)
    for i, x in enumerate(lists):
        idx[i, :len(x)] = x
    log_case(f"token index subset G={G}")
    p = problem(w, q, k, v, g, tok_idx=idx.reshape(-1), n_idx=nidx, idx_stride=stride)
    ref, ref_lse = oracle.attention_rows(p, oracle.all_rows(p), nthreads=8)
    out, lse = run_decode(w, q, k, v, g, split_tokens=256, token_idx=to_dev(idx), n_idx=to_dev(nidx))
    check(out, lse, ref, ref_lse)


@pytest.mark.parametrize("D,maxc,misaligned,rows", [(128, 9, False, 37), (128, 300, False, 37), (64, 300, False, 37),
                                                    (4, 70, False, 37), (37, 40, False, 37), (128, 50, True, 37),
                                                    (128, 12, False, 700), (64, 200, False, 600)])
def test_merge_lse_of_oracle_partials(D, maxc, misaligned, rows):
    """attn_merge_lse on random partials: empty rows, empty partials holding
    NaN outputs (they must be ignored), rows longer than one pass of the
    single-pass kernel, odd head sizes, an output not 16-byte aligned (the
    general kernel), and more than 512 rows (the single-pass kernel's
    serial combine instead of its butterfly)."""
    rng = np.random.default_rng(3 + D + maxc)
    counts = rng.integers(0, maxc, size=rows)
    counts[0] = 0
    rss = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    n = int(rss[-1])
    m = rng.normal(0, 3, n)
    l = rng.uniform(0.5, 40, n)
    l[rng.random(n) < 0.1] = 0.0          # empty chunks
    o = rng.normal(0, 1, (n, D))
    o[l == 0.0] = np.nan
    log_case(f"merge of oracle partials D={D} max count={maxc} misaligned={misaligned} rows={rows}")
    out_buf = torch.empty(rows * D + 1, dtype=torch.float32, device=DEV)
    out_t = out_buf[1:].view(rows, D) if misaligned else out_buf[:rows * D].view(rows, D)
    out, lse = pkg.attn_merge_lse(to_dev(o.astype(np.float32)), to_dev(m.astype(np.float32)),
                                  to_dev(l.astype(np.float32)), to_dev(rss), out=out_t,
                                  lse=torch.empty(rows, dtype=torch.float32, device=DEV))
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    lse = lse.cpu().numpy()
    for r in range(rows):
        s0, s1 = rss[r], rss[r + 1]
        keep = l[s0:s1] > 0
        ro, rl = oracle.merge(m[s0:s1][keep].astype(np.float32).astype(np.float64),
                              l[s0:s1][keep].astype(np.float32).astype(np.float64),
                              o[s0:s1][keep].astype(np.float32).astype(np.float64))
        assert np.abs(out[r] - ro).max() <= 1e-5
        if math.isinf(rl):
            assert math.isinf(lse[r]) and lse[r] < 0
        else:
            assert abs(lse[r] - rl) <= 1e-5


def _full_size_all_rows(name, **over):
    """A full-size workload in the benchmark's launch configuration, every output row compared
    with the oracle; then the property that the softmax weights sum to one: a constant V comes
    back unchanged, and lse does not depend on V."""
    w = synth.workload(name, **over)
    q, k, v, g = synth.generate(w)
    log_case(f"{name} full size, split {w.split_tokens}")
    out, lse = run_decode(w, q, k, v, g, split_tokens=w.split_tokens)
    p = problem(w, q, k, v, g)
    ref, ref_lse = oracle_all_rows(p)
    check(out, lse, ref, ref_lse)
    del p, v
    vc = np.full(k.shape, 0x3FC0, dtype=np.uint16)  # bf16 1.5 everywhere
    out_c, lse_c = run_decode(w, q, k, vc, g, split_tokens=w.split_tokens)
    live = np.repeat(g.lens > 0, w.QH)
    assert np.abs(out_c[live] - 1.5).max() <= 1e-5
    assert np.array_equal(lse_c, lse)


def test_gqa32k_full_size_all_rows():
    """The 16 x 8 x 8 x 128 x 32768 bf16 workload."""
    _full_size_all_rows("gqa32k")


def test_dense128k_full_size_all_rows():
    """The 4 x 8 x 8 x 128 x 131072 bf16 workload the benchmark's headline line times."""
    _full_size_all_rows("dense128k")


def test_ragged_full_size_all_rows():
    """The 32-sequence ragged batch (512..131072 tokens, head-major packed cache)."""
    _full_size_all_rows("ragged")


@pytest.mark.parametrize("name", ["gqa32k", "dense128k"])
def test_one_kv_head_share_full_size_all_rows(name):
    """One GPU's share of a split over 8 GPUs by KV heads (KH = 1, the rest of the shape as named),
    in the library's default launch."""
    _full_size_all_rows(name, KH=1, split_tokens=0)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_reused_workspace_after_longer_rows(out_dtype):
    """The merge's first slot loads run ahead of a row's own chunk count, so
    slots past that count may still hold live partials of an earlier call on
    the same workspace: a call over full-length rows followed by one over
    shorter rows (prefixes of the same K/V, the same workspace and chunk
    layout) must give exactly the shorter rows' result."""
    import dataclasses
    full = 4096
    w = synth.workload("gqa32k", B=4, KH=2, lens=np.full(4, full, np.int32), split_tokens=256, seed=141)
    q, k, v, g = synth.generate(w)
    qd = to_dev(q.reshape(-1)).view(w.B, w.QH, w.D)
    kd, vd = to_dev(k), to_dev(v)
    geom = dev_geom(g)
    lse = torch.empty((w.B, w.QH), dtype=torch.float32, device=DEV)
    p = pkg.prepare_decode(qd, kd, vd, geom, w.G, lse=lse, out_dtype=out_dtype, split_tokens=w.split_tokens)
    log_case(f"reused workspace: full-length call ({out_dtype})")
    p()
    torch.cuda.synchronize()
    ref_full, _ = oracle.attention_rows(problem(w, q, k, v, g), [(0, 0), (3, w.QH - 1)])
    got_full = p.out.float().cpu().numpy().reshape(w.B * w.QH, w.D)[[0, 4 * w.QH - 1]]
    assert np.abs(got_full - ref_full).max() <= TOL + (np.abs(ref_full).max() * 2.0 ** -9)
    short = np.array([100, 0, full, 1500], np.int32)
    geom.seq_lens.copy_(torch.from_numpy(short))
    log_case(f"reused workspace: shorter rows {short.tolist()} ({out_dtype})")
    p()
    torch.cuda.synchronize()
    g2 = dataclasses.replace(g, lens=short)
    pr = problem(w, q, k, v, g2)
    ref, ref_lse = oracle.attention_rows(pr, oracle.all_rows(pr), nthreads=8)
    check(p.out.float().cpu().numpy().reshape(w.B * w.QH, w.D), lse.cpu().numpy().reshape(-1), ref, ref_lse,
          bf16_out=out_dtype == torch.bfloat16)


@pytest.mark.parametrize("fill", ["random", "ones", "zeros"])
def test_workspace_needs_no_clearing(fill):
    """The merge inside the decode launch counts arrivals per (b, kh) in the workspace.  Whatever
    the workspace holds before a call (random bytes, all ones, zeros), the result equals the
    oracle's and a second call on the same workspace reproduces it bit for bit."""
    lens = np.array([3000, 65, 0, 4097], np.int32)
    w = synth.workload("gqa32k", B=4, KH=4, G=8, lens=lens, layout="token_major", seed=171)
    q, k, v, g = synth.generate(w)
    qd = to_dev(q.reshape(-1)).view(w.B, w.QH, w.D)
    kd, vd = to_dev(k), to_dev(v)
    lse = torch.empty((w.B, w.QH), dtype=torch.float32, device=DEV)
    p = pkg.prepare_decode(qd, kd, vd, dev_geom(g), w.G, lse=lse, split_tokens=128)
    ws = p.workspace
    gen = torch.Generator(device="cpu").manual_seed(5)
    if fill == "random":
        ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, generator=gen))
    elif fill == "ones":
        ws.fill_(255)
    else:
        ws.zero_()
    log_case(f"workspace filled with {fill}")
    p()
    torch.cuda.synchronize()
    a_out, a_lse = p.out.cpu().numpy().copy(), lse.cpu().numpy().copy()
    pr = problem(w, q, k, v, g)
    ref, ref_lse = oracle.attention_rows(pr, oracle.all_rows(pr), nthreads=8)
    check(a_out.reshape(w.B * w.QH, w.D), a_lse.reshape(-1), ref, ref_lse)
    p()
    torch.cuda.synchronize()
    check(p.out.cpu().numpy().reshape(w.B * w.QH, w.D), lse.cpu().numpy().reshape(-1), ref, ref_lse)
    assert np.array_equal(a_out, p.out.cpu().numpy()) and np.array_equal(a_lse, lse.cpu().numpy())


def test_interleaved_calls_sharing_one_workspace():
    """Two decode problems of different shapes take turns on one workspace tensor (their counter
    arrays sit at different offsets of it and the partials of one overwrite the other's), each
    several times, with the profiled entry point in between: every call reproduces its first
    result bit for bit, and the first results match the oracle."""
    probs = []
    for lens, KH, split, seed in ((np.array([5000, 70, 2049], np.int32), 2, 256, 181),
                                  (np.array([900, 40000], np.int32), 4, 512, 182)):
        w = synth.workload("gqa32k", B=len(lens), KH=KH, G=8, lens=lens, layout="token_major", seed=seed)
        q, k, v, g = synth.generate(w)
        probs.append((w, q, k, v, g, split))
    need = 0
    preps = []
    for w, q, k, v, g, split in probs:
        qd = to_dev(q.reshape(-1)).view(w.B, w.QH, w.D)
        lse = torch.empty((w.B, w.QH), dtype=torch.float32, device=DEV)
        preps.append((qd, to_dev(k), to_dev(v), dev_geom(g), lse))
    for (w, *_rest, split), (qd, kd, vd, geom, lse) in zip(probs, preps):
        a = pkg.prepare_decode(qd, kd, vd, geom, w.G, lse=lse, split_tokens=split)
        need = max(need, a.workspace.numel())
    ws = torch.full((need,), 0x5A, dtype=torch.uint8, device=DEV)
    calls = [pkg.prepare_decode(qd, kd, vd, geom, w.G, lse=lse, split_tokens=split, workspace=ws)
             for (w, *_rest, split), (qd, kd, vd, geom, lse) in zip(probs, preps)]
    first = []
    for i, c in enumerate(calls):
        log_case(f"shared workspace, problem {i}")
        c()
        torch.cuda.synchronize()
        first.append((c.out.cpu().numpy().copy(), preps[i][4].cpu().numpy().copy()))
    for (w, q, k, v, g, _), (o, l) in zip(probs, first):
        pr = problem(w, q, k, v, g)
        ref, ref_lse = oracle.attention_rows(pr, oracle.all_rows(pr), nthreads=8)
        check(o.reshape(w.B * w.QH, w.D), l.reshape(-1), ref, ref_lse)
    events = [None, None, None]
    for r in range(6):
        i = r % 2
        if r == 3:
            calls[i].profiled(events)
        else:
            calls[i]()
        torch.cuda.synchronize()
        assert np.array_equal(calls[i].out.cpu().numpy(), first[i][0]), f"call {r} (problem {i})"
        assert np.array_equal(preps[i][4].cpu().numpy(), first[i][1]), f"call {r} (problem {i})"


def test_many_workers_per_sequence_and_whole_sequences_per_worker():
    """split_tokens = 32 cuts one long sequence over hundreds of workers (hundreds of partials
    folded by the last arrival), while a batch of short sequences puts several whole sequences in
    one worker's range (their outputs written directly, no partial)."""
    lens = np.array([60000, 40, 33, 1, 200, 96], np.int32)
    w = synth.workload("gqa32k", B=len(lens), KH=1, G=8, lens=lens, layout="head_major", seed=172)
    q, k, v, g = synth.generate(w)
    pr = problem(w, q, k, v, g)
    ref, ref_lse = oracle.attention_rows(pr, oracle.all_rows(pr), nthreads=8)
    for split in (32, 0, 1 << 20):
        log_case(f"split {split}")
        out, lse = run_decode(w, q, k, v, g, split_tokens=split)
        check(out, lse, ref, ref_lse)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_unaligned_output(out_dtype):
    """out may start at any element: the merge's stores fall back to element stores when out is
    not aligned for vector stores; the values equal the aligned call's bit for bit."""
    w = synth.workload("gqa32k", B=2, KH=2, L=3000, seed=173)
    q, k, v, g = synth.generate(w)
    qd = to_dev(q.reshape(-1)).view(w.B, w.QH, w.D)
    kd, vd, geom = to_dev(k), to_dev(v), dev_geom(g)
    n = w.B * w.QH * w.D
    big = torch.zeros(n + 1, dtype=out_dtype, device=DEV)
    odd = big[1:].view(w.B, w.QH, w.D)
    log_case(f"unaligned out {out_dtype}")
    a, _ = pkg.attn_decode_splitkv(qd, kd, vd, geom, w.G, out_dtype=out_dtype)
    b, _ = pkg.attn_decode_splitkv(qd, kd, vd, geom, w.G, out=odd)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("splits", [1, 3, 40])
def test_fixed_splits_schedule_matches_oracle(splits):
    """The unbalanced schedule kept for comparison (every (b, kh) cut into the same number of
    splits, one worker each): sequences shorter than the split count, an empty one and a long
    one, bf16 and int8."""
    lens = np.array([5000, 17, 0, 900, 1], np.int32)
    w = synth.workload("gqa32k", B=len(lens), KH=2, G=8, lens=lens, layout="token_major", seed=174)
    q, k, v, g = synth.generate(w)
    pr = problem(w, q, k, v, g)
    ref, ref_lse = oracle.attention_rows(pr, oracle.all_rows(pr), nthreads=8)
    log_case(f"fixed splits {splits} bf16")
    out, lse = run_decode(w, q, k, v, g, fixed_splits=splits)
    check(out, lse, ref, ref_lse)
    geom = dev_geom(g)
    kc, ks = pkg.kv_quant_int8(to_dev(k), geom, 64)
    vc, vs = pkg.kv_quant_int8(to_dev(v), geom, 0)
    torch.cuda.synchronize()
    p8 = problem(w, q, kc.cpu().numpy(), vc.cpu().numpy(), g, k_scale=ks.cpu().numpy(), k_part=64,
                 k_scale_stride=-(-int(g.max_len) // 64), v_scale=float(vs.item()))
    ref8, ref8_lse = oracle.attention_rows(p8, oracle.all_rows(p8), nthreads=8)
    log_case(f"fixed splits {splits} int8")
    qd = to_dev(q.reshape(-1)).view(w.B, w.QH, w.D)
    lse8 = torch.empty((w.B, w.QH), dtype=torch.float32, device=DEV)
    o8, _ = pkg.attn_decode_splitkv(qd, kc, vc, geom, w.G, lse=lse8, k_scale=ks, k_part_tokens=64,
                                    v_scale=float(vs.item()), fixed_splits=splits)
    torch.cuda.synchronize()
    check(o8.cpu().numpy().reshape(w.B * w.QH, w.D), lse8.cpu().numpy().reshape(-1), ref8, ref8_lse)


def test_indexed_full_grid_uses_the_xcd_weighted_split():
    """Kept-token attention whose lists hold every position of 4 x 8 lanes of 32768 tokens: enough
    tiles for the whole grid under the default cache policy, so the XCD-weighted work split runs
    (streaming launches split equally, and gathered rows keep the default policy).  Listing every
    position makes it dense attention: every output row and lse against the oracle's."""
    L = 32768
    w = synth.workload("gqa32k", B=4, KH=8, G=8, lens=np.full(4, L, np.int32), layout="head_major", seed=176)
    q, k, v, g = synth.generate(w)
    idx = np.tile(np.arange(L, dtype=np.int32), (w.B * w.KH, 1))
    nk = np.full(w.B * w.KH, L, np.int32)
    log_case("indexed, every position listed, full grid")
    out, lse = run_decode(w, q, k, v, g, token_idx=to_dev(idx), n_idx=to_dev(nk))
    ref, ref_lse = oracle_all_rows(problem(w, q, k, v, g))
    check(out, lse, ref, ref_lse)
