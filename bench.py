#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

Headline: bf16 GQA decode at 128K KV (B=4 sequences, 8 KV heads, G=8 query
heads per KV head, head dim 128, 131072 tokens each, split-KV over the
library's default work split, partials merged by log-sum-exp inside the same
launch).  One step = one attn_decode_splitkv call over inputs already resident
in HBM.  Prints one JSON line: KV GB/s (value), us/step (mean of back-to-back
steps, and the median and minimum of single steps timed one by one), fraction
of HBM peak and of a measured read-only HBM probe, the roofline of the decode
kernel, the CPU oracle baseline and, unless --headline-only, the other
workloads (32K GQA, ragged batch with the balanced and the unbalanced
schedules, INT8 KV and its scheme table, a paged cache, multi-row speculative
steps, OAM token dropping on bf16 and INT8 caches, and block-granular
selection).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, vendor figure
METRIC = "decode-attention KV GB/s (% of MI355X HBM peak) + µs/step at 128K KV"
PMC_SUMMARY = os.path.join(ROOT, "profiles", "decode_mfma_dense128k_pmc.txt")
# the decode kernel, the header it inlines and the build script (its compiler flags); counters
# taken on other sources are stale
DECODE_SOURCES = [os.path.join(ROOT, "long_context_decode_gqa_amd", f)
                  for f in ("csrc/decode_mfma.hip", "csrc/common.hpp", "build.py")]


# ------------------------------------------------------------------ byte/flop accounting

def gqa_cache_elements(kv_heads: int, head_dim: int, seq_len: int) -> int:
    """K plus V cache entries of one sequence (the GQA example's 2 x heads x dim x len)."""
    return 2 * kv_heads * head_dim * seq_len


def decode_eq_elements(DB: int, KH: int, G: int, Hsz: int, KVSL: int) -> int:
    """Decode bytes at one byte per element: 2 x DB x KH x Hsz x (G + KVSL) (Q/O plus the KV cache)."""
    return 2 * DB * KH * Hsz * (G + KVSL)


def decode_eq_flops(DB: int, QH: int, KVSL: int, Hsz: int) -> int:
    """Decode FLOPs: 4 x DB x QH x KVSL x Hsz."""
    return 4 * DB * QH * KVSL * Hsz


def kv_bytes(total_tokens: int, KH: int, D: int, elem_bytes: int) -> int:
    """Bytes of K plus V streamed for `total_tokens` cached tokens of every KV head."""
    return 2 * total_tokens * KH * D * elem_bytes


def partial_bytes(n_partials: int, D: int) -> int:
    """Split-KV partial triples written by the decode kernel: o (D floats), m and l."""
    return n_partials * (D + 2) * 4


# ------------------------------------------------------------------ helpers

def host_threads() -> int:
    """Host cores this job may use: the cores it may run on, capped by the CPU share the machine
    grants it (OMP_NUM_THREADS where set); the CPU baseline uses every one of them."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    share = os.environ.get("OMP_NUM_THREADS", "")
    if share.isdigit() and int(share) > 0:
        n = min(n, int(share))
    return max(1, n)


def sources_sha256(paths) -> str:
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_pmc_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; None otherwise."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    kv = {}
    for line in open(PMC_SUMMARY):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            kv[key.strip()] = val.strip()
    if kv.get("kernel_sources_sha256") != sources_sha256(DECODE_SOURCES):
        return None
    try:
        return int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


class Timer:
    """HIP events around K steps on the current stream, plus per-phase events."""

    def __init__(self, torch, steps):
        self.torch = torch
        self.start = torch.cuda.Event(enable_timing=True)
        self.end = torch.cuda.Event(enable_timing=True)
        self.phase = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for evs in self.phase:          # materialise the events so their handles exist
            for e in evs:
                e.record()
        torch.cuda.synchronize()


def time_calls(torch, fn, steps, warmup):
    """Mean ms per call of fn (launches on the current stream), between two events."""
    for _ in range(warmup):
        fn()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(steps):
        fn()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def to_dev(torch, a, dev):
    import numpy as np
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def dev_geom(pkg, torch, g, dev):
    return pkg.KVGeometry(g.B, g.KH, g.D, int(g.max_len), torch.from_numpy(g.lens).to(dev),
                          torch.from_numpy(g.seq_offset).to(dev), g.stride_h, g.stride_t)


def time_decode(torch, prepared, steps, warmup):
    """Returns a dict of ms: `step` = mean of `steps` plain calls back to back between two events;
    `decode` = mean duration of the decode launch, from a second run of `steps` calls through the
    profiled entry point, whose events sit on the calls' stream around each launch (bf16/int8 KV:
    the merge runs inside the decode launch, so that launch is the whole step, and the profiled
    entry point's merge phase is empty: its two events only measure their own gap, about 4.5 us,
    which is left out); `median` / `min` = of those per-call decode launch durations."""
    for _ in range(warmup):
        prepared()
    t = Timer(torch, steps)
    torch.cuda.synchronize()
    t.start.record()
    for _ in range(steps):
        prepared()
    t.end.record()
    torch.cuda.synchronize()
    total = t.start.elapsed_time(t.end)
    for i in range(steps):
        prepared.profiled(t.phase[i])
    torch.cuda.synchronize()
    dk = [e[0].elapsed_time(e[1]) for e in t.phase]
    per = sorted(dk)
    return {"step": total / steps, "decode": sum(dk) / steps, "median": per[len(per) // 2], "min": per[0]}


# ------------------------------------------------------------------ workloads

def grid_slots(pkg, w) -> int:
    """Decode workers the balanced split runs for a bf16 workload of this shape on this GPU (four-wave
    workers, eight waves per compute unit)."""
    import torch
    n = torch.cuda.get_device_properties(0).multi_processor_count
    return n * 8 // 4


def bench_dense(pkg, torch, synth, name, steps, warmup, dev, unbalanced=False, **over):
    w = synth.workload(name, **over)
    q, k, v, g = synth.generate(w, nthreads=host_threads())
    qd = to_dev(torch, q.reshape(-1), dev).view(w.B, w.QH, w.D)
    kd, vd = to_dev(torch, k, dev), to_dev(torch, v, dev)
    del k, v
    geom = dev_geom(pkg, torch, g, dev)
    p = pkg.prepare_decode(qd, kd, vd, geom, w.G, split_tokens=w.split_tokens)
    t = time_decode(torch, p, steps, warmup)
    tokens = w.kv_tokens()
    kvb = kv_bytes(tokens, w.KH, w.D, 2)
    # the bytes the step must move: K/V once, Q in and out (bf16 Q, fp32 out)
    algo = kvb + w.B * w.QH * w.D * (2 + 4)
    res = dict(w=w, q=q, g=g, t=t, ms=t["step"], decode_ms=t["decode"], kv_bytes=kvb,
               decode_algo_bytes=algo, tokens=tokens, split=p.split_tokens)
    if unbalanced:
        # The unbalanced schedules on the same inputs, every (b, kh) in the same number of equal
        # splits whatever its length: one worker per (b, kh); as many splits as fill the grid once;
        # and as many as cut the longest sequence into pieces of the balanced range (flash-decoding
        # style, the split count chosen for the longest sequence).
        lanes = w.B * w.KH
        W = grid_slots(pkg, w)
        tiles = [-(-int(L) // 32) for L in w.lens]
        T = w.KH * sum(tiles)
        fill = max(1, -(-W // lanes))
        longest = max(1, -(-max(tiles) * W // T))
        for tag, S in (("per_sequence", 1), (f"fixed_{fill}_splits", fill), (f"fixed_{longest}_splits", longest)):
            pu = pkg.prepare_decode(qd, kd, vd, geom, w.G, fixed_splits=S)
            res.setdefault("unbalanced", {})[tag] = time_decode(torch, pu, max(3, steps // 2), 2)
            res["unbalanced"][tag]["splits_per_sequence"] = S
            del pu
    return res


def summary(r, extra=None, probe_gbs=None):
    d = {"us_per_step": round(r["ms"] * 1e3, 2), "kv_gbs": round(r["kv_bytes"] / r["ms"] / 1e6, 1),
         "frac_of_peak": round(r["kv_bytes"] / r["ms"] / 1e6 / HBM_PEAK_GBS, 4),
         "us_per_step_median": round(r["t"]["median"] * 1e3, 2), "us_per_step_min": round(r["t"]["min"] * 1e3, 2),
         "decode_kernel_us": round(r["decode_ms"] * 1e3, 2),
         "kernel_kv_gbs": round(r["kv_bytes"] / r["decode_ms"] / 1e6, 1),
         "kernel_frac_of_peak": round(r["kv_bytes"] / r["decode_ms"] / 1e6 / HBM_PEAK_GBS, 4)}
    if probe_gbs:
        d["frac_of_probe"] = round(r["kv_bytes"] / r["ms"] / 1e6 / probe_gbs, 4)
    if "split" in r:
        d["split_tokens"] = r["split"]
    if extra:
        d.update(extra)
    return d


def bench_int8(pkg, torch, synth, steps, warmup, dev):
    """INT8 KV decode at 128K: the configured workload (bf16 query, K per 64-token partition, V per
    tensor), then the page's scheme table (§6): A = per-row int8 query with 64- or 128-token K
    partitions, B = per-row query with one K scale, baseline = static per-tensor query, K and V.
    Each scheme reports its step time and its output's relative error against the bf16 path."""
    w = synth.workload("int8_128k")
    q, k, v, g = synth.generate(w, nthreads=host_threads())
    geom = dev_geom(pkg, torch, g, dev)
    kd, vd = to_dev(torch, k, dev), to_dev(torch, v, dev)
    del k, v
    qd = to_dev(torch, q.reshape(-1), dev).view(w.B, w.QH, w.D)
    ref = pkg.prepare_decode(qd, kd, vd, geom, w.G, split_tokens=w.split_tokens)
    ref()
    k_codes = {part: pkg.kv_quant_int8(kd, geom, part) for part in (64, 128, 0)}
    vc, vs = pkg.kv_quant_int8(vd, geom, 0)
    # cache-write-time quantisation (not part of a decode step): K per 64-token partition (one read,
    # one write) and V per tensor (a max pass, then a code pass: two reads, one write)
    elems = w.kv_tokens() * w.KH * w.D
    kc64, ks64 = k_codes[64]
    t_kq = time_calls(torch, lambda: pkg.kv_quant_int8(kd, geom, 64, codes=kc64, scales=ks64), steps, warmup)
    t_vq = time_calls(torch, lambda: pkg.kv_quant_int8(vd, geom, 0, codes=vc, scales=vs), steps, warmup)
    quant = {"k_partition64_us": round(t_kq * 1e3, 2),
             "k_partition64_gbs": round((elems * 3 + ks64.numel() * 4) / t_kq / 1e6, 1),
             "v_tensor_us": round(t_vq * 1e3, 2),
             "v_tensor_gbs": round((elems * 5 + 4) / t_vq / 1e6, 1)}
    # static per-tensor query scale, calibrated once on this query with the library's quantiser
    qgeom = pkg.KVGeometry(w.B, w.QH, w.D, 1, torch.ones(w.B, dtype=torch.int32, device=dev),
                           torch.arange(w.B, dtype=torch.int64, device=dev) * (w.QH * w.D), w.D, w.D)
    _, q_static = pkg.kv_quant_int8(qd.reshape(-1), qgeom, 0)
    torch.cuda.synchronize()
    ref_out = ref.out.clone()
    del kd, vd, ref
    vs_f, qs_f = float(vs.item()), float(q_static.item())

    def prep(part, q_quant):
        kc, ks = k_codes[part]
        return pkg.prepare_decode(qd, kc, vc, geom, w.G, k_scale=ks, k_part_tokens=part, v_scale=vs_f,
                                  split_tokens=w.split_tokens, q_quant=q_quant, q_scale=qs_f)

    tokens = w.kv_tokens()
    p = prep(64, pkg.QUANT_EXACT)
    # the quantisation passes just wrote 1.5 GiB and the host then idled on the scale read: the
    # first steps after that run slow (after 50 warm-up steps the mean was still 6-11 us above the
    # same configuration timed again later as the scheme "bf16_query_k64"), so the untimed warm-up
    # is 300 steps (about 50 ms)
    t = time_decode(torch, p, steps, max(2 * warmup, 300))
    kvb = kv_bytes(tokens, w.KH, w.D, 1) + k_codes[64][1].numel() * 4 + 4
    schemes = {}
    for name, part, qq in (("A_k64", 64, pkg.QUANT_ROW), ("A_k128", 128, pkg.QUANT_ROW),
                           ("B", 0, pkg.QUANT_ROW), ("baseline", 0, pkg.QUANT_STATIC),
                           ("bf16_query_k64", 64, pkg.QUANT_EXACT)):
        ps = prep(part, qq)
        ts = time_decode(torch, ps, steps, warmup)
        ms_s, dk_s = ts["step"], ts["decode"]
        err = float(torch.linalg.norm(ps.out - ref_out) / torch.linalg.norm(ref_out))
        b = kv_bytes(tokens, w.KH, w.D, 1) + k_codes[part][1].numel() * 4 + 4
        schemes[name] = {"us_per_step": round(ms_s * 1e3, 2), "decode_kernel_us": round(dk_s * 1e3, 2),
                         "kv_gbs": round(b / ms_s / 1e6, 1), "rel_err_vs_bf16": round(err, 5)}
        del ps
    return dict(t=t, ms=t["step"], decode_ms=t["decode"], kv_bytes=kvb, split=p.split_tokens,
                schemes=schemes,
                quant=quant)


def bench_paged(pkg, torch, synth, steps, warmup, dev, page_tokens=64, layout="head_major"):
    """The 128K bf16 decode over a paged cache: the same K/V rows moved into a pool of
    head-major ([pages][KH][page_tokens][D]) or token-major ([pages][page_tokens][KH][D]) pages
    in scrambled order, read through a block table.  Pool construction is setup, outside the
    timed region."""
    w = synth.workload("dense128k")
    q, k, v, g = synth.generate(w, nthreads=host_threads())
    B, KH, D, L, P = w.B, w.KH, w.D, int(w.lens[0]), page_tokens
    npg = L // P
    gen = torch.Generator().manual_seed(12)
    perm = torch.randperm(B * npg, generator=gen).to(dev)

    def pool_of(x):
        t = to_dev(torch, x, dev).view(B, KH, npg, P, D)
        if layout == "head_major":
            t = t.permute(0, 2, 1, 3, 4).reshape(B * npg, KH, P, D)
        else:
            t = t.permute(0, 2, 3, 1, 4).reshape(B * npg, P, KH, D)
        pool = torch.empty_like(t)
        pool[perm] = t                      # logical page i of the batch lives at pool page perm[i]
        return pool.reshape(-1)

    kp, vp = pool_of(k), pool_of(v)
    del k, v
    table = perm.view(B, npg).to(torch.int32).contiguous()
    stride_h, stride_t = (P * D, D) if layout == "head_major" else (D, KH * D)
    geom = pkg.KVGeometry(B, KH, D, L, torch.full((B,), L, dtype=torch.int32, device=dev), None, stride_h, stride_t,
                          block_table=table, page_tokens=P, page_stride=P * KH * D)
    qd = to_dev(torch, q.reshape(-1), dev).view(w.B, w.QH, w.D)
    p = pkg.prepare_decode(qd, kp, vp, geom, w.G, split_tokens=w.split_tokens)
    t = time_decode(torch, p, steps, warmup)
    res = dict(t=t, ms=t["step"], decode_ms=t["decode"], kv_bytes=kv_bytes(w.kv_tokens(), KH, D, 2),
               split=p.split_tokens)
    if layout == "head_major":
        # OAM selection (top 4096 of the 128K tokens) over the same pool, value term cached
        vlog = pkg.oam_value_lognorm(vp, geom, 1e-6)
        sel = pkg.prepare_oam(qd, kp, geom, w.G, 4096, vlog=vlog, beta=1.0, eps=1e-6)
        res["oam_select_ms"] = time_calls(torch, sel, steps, warmup)
        res["value_lognorm_ms"] = time_calls(torch, lambda: pkg.oam_value_lognorm(vp, geom, 1e-6, vlog=vlog),
                                             steps, warmup)
    return res


def bench_tiny(pkg, torch, synth, steps, warmup, dev):
    """The tiny fp32 case (B1, KH1, G4, D64, L1024): 512 KiB of K/V, so a step is launch-bound, not a
    bandwidth point.  Unsplit and in 4 chunks of 256 + merge; warm (back to back) and cold (a 512 MiB
    write between calls)."""
    w = synth.workload("tiny")
    q, k, v, g = synth.generate(w)
    geom = dev_geom(pkg, torch, g, dev)
    qd = to_dev(torch, q.reshape(-1), dev).view(w.B, w.QH, w.D)
    kd, vd = to_dev(torch, k, dev), to_dev(torch, v, dev)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    res = {"kv_bytes": int(w.B * w.KH * int(w.lens[0]) * w.D * 4 * 2)}
    for name, split in (("unsplit", 1024), ("split4", 256)):
        p = pkg.prepare_decode(qd, kd, vd, geom, w.G, split_tokens=split)
        res[f"{name}_warm_us"] = round(time_calls(torch, p, steps, warmup) * 1e3, 2)
        cold = []
        for _ in range(max(3, steps // 2)):
            flush.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            p()
            e1.record()
            torch.cuda.synchronize()
            cold.append(e0.elapsed_time(e1))
        res[f"{name}_cold_us"] = round(sorted(cold)[len(cold) // 2] * 1e3, 2)
    return res


def bench_multirow(pkg, torch, synth, steps, warmup, dev, R):
    """The 128K bf16 decode with R query rows per sequence (speculative verification: each step
    checks R tokens).  Same K/V bytes as one row; G * R rows of a KV head share each load."""
    w = synth.workload("dense128k")
    _, k, v, g = synth.generate(w, nthreads=host_threads())
    geom = dev_geom(pkg, torch, g, dev)
    kd, vd = to_dev(torch, k, dev), to_dev(torch, v, dev)
    del k, v
    q = synth.fill_q(151, w.B, R * w.QH, w.D, synth.BF16)
    qd = to_dev(torch, q.reshape(-1), dev).view(w.B, R, w.QH, w.D)
    p = pkg.prepare_decode(qd, kd, vd, geom, w.G, split_tokens=w.split_tokens, q_rows=R)
    t = time_decode(torch, p, steps, warmup)
    return dict(t=t, ms=t["step"], decode_ms=t["decode"], kv_bytes=kv_bytes(w.kv_tokens(), w.KH, w.D, 2),
                split=p.split_tokens)


def bench_oam(pkg, torch, synth, steps, warmup, dev):
    """OAM step: score + exact top-K over the cached value log-norms, then exact
    attention over the kept tokens.  Also times the variant that reads V to get
    the norms on the fly."""
    w = synth.workload("oam_128k")
    q, k, v, g = synth.generate(w, nthreads=host_threads())
    geom = dev_geom(pkg, torch, g, dev)
    qd = to_dev(torch, q.reshape(-1), dev).view(w.B, w.QH, w.D)
    kd, vd = to_dev(torch, k, dev), to_dev(torch, v, dev)
    del k, v
    vlog = pkg.oam_value_lognorm(vd, geom, w.eps)          # computed when tokens are appended
    sel = pkg.prepare_oam(qd, kd, geom, w.G, w.top_k, vlog=vlog, beta=w.beta, eps=w.eps)
    sel_fly = pkg.prepare_oam(qd, kd, geom, w.G, w.top_k, v=vd, beta=w.beta, eps=w.eps)
    att = pkg.prepare_decode(qd, kd, vd, geom, w.G, token_idx=sel.idx_out, n_idx=sel.n_kept,
                             split_tokens=w.split_tokens)

    def timed(fn_list, n):
        """(ms per step of the whole list, [ms of each call]): the step time from
        plain back-to-back steps, the split from a second run with events between
        the calls."""
        for _ in range(warmup):
            for f in fn_list:
                f()
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s0.record()
        for _ in range(n):
            for f in fn_list:
                f()
        s1.record()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fn_list) + 1)] for _ in range(n)]
        for i in range(n):
            evs[i][0].record()
            for j, f in enumerate(fn_list):
                f()
                evs[i][j + 1].record()
        torch.cuda.synchronize()
        return s0.elapsed_time(s1) / n, [sum(e[j].elapsed_time(e[j + 1]) for e in evs) / n for j in range(len(fn_list))]

    ms, (t_sel, t_att) = timed([sel, att], steps)
    t_fly, _ = timed([sel_fly], max(3, steps // 2))
    L, KH, D = int(w.lens[0]), w.KH, w.D
    npairs = w.B * KH
    algo = (npairs * L * D * 2 + npairs * L * 4 + 2 * npairs * L * 4 + 2 * npairs * w.top_k * D * 2
            + npairs * w.top_k * 4)
    res = {"us_per_step": round(ms * 1e3, 2), "select_us": round(t_sel * 1e3, 2),
           "kept_attention_us": round(t_att * 1e3, 2), "algorithmic_bytes_per_step": algo,
           "gbs_algorithmic": round(algo / ms / 1e6, 1), "frac_of_peak": round(algo / ms / 1e6 / HBM_PEAK_GBS, 4),
           "select_with_norms_from_v_us": round(t_fly * 1e3, 2), "top_k": w.top_k, "kv_len": L}
    # the kept-token attention alone, warm (back to back: its 64 MiB of gathered rows stay in the
    # 256 MB Infinity Cache) and cold (a 512 MiB write between calls evicts them)
    res["kept_attention_warm_us"] = round(time_calls(torch, att, steps, warmup) * 1e3, 2)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = []
    for _ in range(max(3, steps // 2)):
        flush.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        att()
        e1.record()
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))
    res["kept_attention_cold_us"] = round(sorted(cold)[len(cold) // 2] * 1e3, 2)
    del flush, sel, sel_fly, att
    # the cached value term, computed when tokens are appended (V read once, 4 bytes written per token)
    t_vl = time_calls(torch, lambda: pkg.oam_value_lognorm(vd, geom, w.eps, vlog=vlog), steps, warmup)
    res["value_lognorm_us"] = round(t_vl * 1e3, 2)
    res["value_lognorm_gbs"] = round(npairs * L * (D * 2 + 4) / t_vl / 1e6, 1)
    # The page's §7 stack on the same data: the cache quantised once (K per 64-token partition, V per
    # tensor), OAM scores over the K codes with the value term from the INT8 values, then INT8
    # attention over the kept tokens.
    kc, ks = pkg.kv_quant_int8(kd, geom, 64)
    vc, vs = pkg.kv_quant_int8(vd, geom, 0)
    torch.cuda.synchronize()
    vs_f = float(vs.item())
    del kd, vd
    vlog8 = pkg.oam_value_lognorm(vc, geom, w.eps, v_scale=vs_f)
    sel8 = pkg.prepare_oam(qd, kc, geom, w.G, w.top_k, vlog=vlog8, beta=w.beta, eps=w.eps, k_scale=ks,
                           k_part_tokens=64, v_scale=vs_f)
    att8 = pkg.prepare_decode(qd, kc, vc, geom, w.G, token_idx=sel8.idx_out, n_idx=sel8.n_kept, k_scale=ks,
                              k_part_tokens=64, v_scale=vs_f, split_tokens=w.split_tokens)
    ms8, (t_sel8, t_att8) = timed([sel8, att8], steps)
    # block-granular selection on the same INT8 cache: the best 64 blocks of 64 tokens (as many
    # tokens as the token top-K keeps) by the mean routing score (beta = 0), then attention over them
    nbk = w.top_k // 64
    selb = pkg.prepare_oam(qd, kc, geom, w.G, nbk, vlog=vlog8, beta=0.0, eps=w.eps, k_scale=ks, k_part_tokens=64,
                           v_scale=vs_f, block_tokens=64)
    attb = pkg.prepare_decode(qd, kc, vc, geom, w.G, token_idx=selb.idx_out, n_idx=selb.n_kept, k_scale=ks,
                              k_part_tokens=64, v_scale=vs_f, split_tokens=w.split_tokens)
    msb, (t_selb, t_attb) = timed([selb, attb], steps)
    nparts = -(-L // 64)
    algo8 = (npairs * L * D + npairs * nparts * 4 + npairs * L * 4 + 2 * npairs * L * 4
             + 2 * npairs * w.top_k * D + npairs * w.top_k * 4 + npairs * w.top_k * 4)
    res["int8_stack"] = {"us_per_step": round(ms8 * 1e3, 2), "select_us": round(t_sel8 * 1e3, 2),
                         "kept_attention_us": round(t_att8 * 1e3, 2), "algorithmic_bytes_per_step": algo8,
                         "gbs_algorithmic": round(algo8 / ms8 / 1e6, 1),
                         "frac_of_peak": round(algo8 / ms8 / 1e6 / HBM_PEAK_GBS, 4)}
    res["int8_block_select"] = {"block_tokens": 64, "blocks_kept": nbk, "us_per_step": round(msb * 1e3, 2),
                                "select_us": round(t_selb * 1e3, 2), "kept_attention_us": round(t_attb * 1e3, 2)}
    return res


def hbm_read_probe(pkg, torch, dev, nbytes=4 << 30, reps=20):
    """The library's read-only sweep (attn_util_read: one contiguous chunk per workgroup, sixteen
    non-temporal 16-byte buffer loads per thread in flight, one checksum word per workgroup) over
    nbytes of HBM, timed with events around each launch on the current stream: the achievable read
    bandwidth next to the 8 TB/s vendor figure."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev)
    src.fill_(1.0)
    sink = torch.empty(4096, dtype=torch.float32, device=dev)
    for _ in range(3):
        pkg.util_read(src, sink)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        pkg.util_read(src, sink)
        b.record()
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in ev)
    del src, sink
    torch.cuda.empty_cache()
    return {"bytes": nbytes, "launches": reps, "us_median": round(per[len(per) // 2] * 1e3, 2),
            "gbs_median": round(nbytes / per[len(per) // 2] / 1e6, 1), "gbs_max": round(nbytes / per[0] / 1e6, 1),
            "kernel": "read_kernel (attn_util_read)"}


def cpu_baseline(r, budget_s=10.0):
    """The fp64 oracle on host threads over whole (b, kh) pairs of the headline workload."""
    import numpy as np

    import oracle
    w, q, g = r["w"], r["q"], r["g"]
    import synth
    k = synth.fill(w.seed, synth.T_K, g, nthreads=host_threads())
    v = synth.fill(w.seed, synth.T_V, g, nthreads=host_threads())
    p = oracle.Problem(w.B, w.KH, w.G, w.D, g.lens, g.seq_offset, g.stride_h, g.stride_t, np.ascontiguousarray(q),
                       k, v, 1.0 / math.sqrt(w.D))
    n = host_threads()
    pairs = [(b, kh) for b in range(w.B) for kh in range(w.KH)]
    cpu_count = os.cpu_count()
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = cpu_count
    per_batch = max(1, n // w.G)
    done = 0
    t0 = time.perf_counter()
    # batches of whole (b, kh) pairs, cycling over the workload until about budget_s of CPU work
    while time.perf_counter() - t0 < budget_s:
        i0 = done % len(pairs)
        batch = pairs[i0:i0 + per_batch]
        rows = [(b, kh * w.G + gq) for b, kh in batch for gq in range(w.G)]
        oracle.attention_rows(p, rows, nthreads=n)
        done += len(batch)
    dt = time.perf_counter() - t0
    bytes_done = kv_bytes(int(w.lens[0]) * done, 1, w.D, 2)
    return {"value": round(bytes_done / dt / 1e9, 3), "unit": "GB/s", "cores": n, "os_cpu_count": cpu_count,
            "affinity_cores": affinity, "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "kind": "oracle",
            "seconds": round(dt, 2), "us_per_step_equiv": round(dt / done * len(pairs) * 1e6, 1),
            "sample": f"{done} (sequence, KV head) pair passes ({done / len(pairs):.1f} sweeps of the "
                      f"{len(pairs)} pairs) of the 128K bf16 workload, all {w.G} query heads each, fp64 oracle "
                      f"on {n} host threads, about {budget_s:.0f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--headline-only", action="store_true")
    ap.add_argument("--others", default="tiny,gqa32k,tp8,ragged,int8,oam,paged,multirow",
                    help="comma-separated other workloads to time after the headline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run the library's plain copy kernel over this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the decode path runs on one GPU only (asked for --gpus {args.gpus}); "
              "its sharding over several GPUs is not implemented", file=sys.stderr)
        sys.exit(2)

    import torch

    import long_context_decode_gqa_amd as pkg
    import synth
    if not os.path.exists(pkg._lib.LIB_PATH):
        from long_context_decode_gqa_amd.build import build
        build()
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    K, W = args.steps, args.warmup
    if args.calibrate_copy_mib:
        nbytes = args.calibrate_copy_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(W + K):
            pkg.util_copy(dst, src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": nbytes, "launches": W + K}), flush=True)
        return

    probe = hbm_read_probe(pkg, torch, dev)
    pg = probe["gbs_median"]
    head = bench_dense(pkg, torch, synth, "dense128k", K, W, dev)
    w = head["w"]
    ms = head["ms"]
    value = head["kv_bytes"] / ms / 1e6          # GB/s (1e9 bytes per second)
    # the decode kernel is the whole step (the merge runs inside it): its launch duration from the
    # events around each launch on the calls' stream
    dk_s = head["decode_ms"] / 1e3
    achieved = head["decode_algo_bytes"] / dk_s / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": read_pmc_traffic(),
                "kernel": "decode_mfma_kernel<128, bf16, non-temporal K/V> (decode and merge, one launch)",
                "algorithmic_bytes_per_launch": head["decode_algo_bytes"],
                "avg_launch_us": round(head["decode_ms"] * 1e3, 2),
                "frac_of_probe": round(achieved / pg, 4)}
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms, 4), "us_per_step": round(ms * 1e3, 2), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "us_per_step_median": round(head["t"]["median"] * 1e3, 2), "us_per_step_min": round(head["t"]["min"] * 1e3, 2),
        "frac_of_probe": round(value / pg, 4), "hbm_read_probe": probe,
        "config": {"workload": "gqa_decode_bf16_128k", "batch": w.B, "kv_heads": w.KH, "group_size": w.G,
                   "head_dim": w.D, "kv_len": int(w.lens[0]), "split_tokens": head["split"],
                   "split_chosen_by": "library" if w.split_tokens == 0 else "caller",
                   "kv_bytes_per_step": head["kv_bytes"],
                   "eq6_bytes_per_step": decode_eq_elements(w.B, w.KH, w.G, w.D, int(w.lens[0])) * 2,
                   "flops_per_step": decode_eq_flops(w.B, w.QH, int(w.lens[0]), w.D)},
        "phases_us": {"decode": round(head["decode_ms"] * 1e3, 2),
                      "launches_per_step": 1},
        "roofline": roofline,
    }
    if not args.headline_only:
        others = {}
        todo = set(x.strip() for x in args.others.split(",") if x.strip())
        if "gqa32k" in todo:
            r = bench_dense(pkg, torch, synth, "gqa32k", max(5, K // 2), W, dev)
            others["gqa32k_bf16"] = summary(r, probe_gbs=pg)
            del r
        if "tiny" in todo:
            others["tiny_fp32"] = bench_tiny(pkg, torch, synth, K, W, dev)
        if "tp8" in todo:
            # one GPU's share of a tensor-parallel split over 8 GPUs by KV heads (KH = 8 -> 1 per GPU):
            # the same per-head work at 1/8 of the bytes, where fixed costs weigh more
            for name in ("gqa32k", "dense128k"):
                r = bench_dense(pkg, torch, synth, name, max(5, K // 2), W, dev, KH=1, split_tokens=0)
                others[f"{name}_tp8_share_kh1"] = summary(r, {"kv_heads": 1, "batch": int(r["w"].B)}, probe_gbs=pg)
                del r
        if "ragged" in todo:
            r = bench_dense(pkg, torch, synth, "ragged", max(5, K // 2), W, dev, unbalanced=True)
            unb = {tag: {"us_per_step": round(t["step"] * 1e3, 2), "us_per_step_median": round(t["median"] * 1e3, 2),
                         "splits_per_sequence": t["splits_per_sequence"],
                         "balanced_speedup": round(t["step"] / r["ms"], 3)}
                   for tag, t in r["unbalanced"].items()}
            others["ragged_bf16"] = summary(r, {"total_kv_tokens_per_head": r["tokens"],
                                                 "lens_min": int(r["w"].lens.min()),
                                                 "lens_max": int(r["w"].lens.max()),
                                                 "unbalanced_schedules": unb}, probe_gbs=pg)
            del r
        if "int8" in todo:
            try:
                r = bench_int8(pkg, torch, synth, K, W, dev)
                others["int8_128k"] = summary(r, probe_gbs=pg)
                others["int8_128k_schemes"] = r["schemes"]
                others["int8_128k_quantisation"] = r["quant"]
            except pkg.AttnError as e:
                others["int8_128k"] = {"error": str(e)}
        if "multirow" in todo:
            for R in (2, 4, 8):
                r = bench_multirow(pkg, torch, synth, max(5, K // 2), W, dev, R)
                others[f"multirow_128k_bf16_R{R}"] = summary(r, {"query_rows": R,
                                                                 "us_per_query_row": round(r["ms"] * 1e3 / R, 2)})
                del r
        if "paged" in todo:
            for lay in ("head_major", "token_major"):
                r = bench_paged(pkg, torch, synth, max(5, K // 2), W, dev, layout=lay)
                extra = {"page_tokens": 64}
                if "oam_select_ms" in r:
                    extra["oam_select_top4096_us"] = round(r["oam_select_ms"] * 1e3, 2)
                    extra["value_lognorm_us"] = round(r["value_lognorm_ms"] * 1e3, 2)
                others[f"paged_128k_bf16_{lay}"] = summary(r, extra)
                del r
        if "oam" in todo:
            try:
                others["oam_128k"] = bench_oam(pkg, torch, synth, max(5, K // 2), W, dev)
                o = others["oam_128k"]
                o["speedup_vs_dense_128k"] = round(ms * 1e3 / o["us_per_step"], 3)
                o["int8_stack"]["speedup_vs_dense_128k"] = round(ms * 1e3 / o["int8_stack"]["us_per_step"], 3)
                o["int8_block_select"]["speedup_vs_dense_128k"] = round(
                    ms * 1e3 / o["int8_block_select"]["us_per_step"], 3)
            except pkg.AttnError as e:
                others["oam_128k"] = {"error": str(e)}
        line["other_workloads"] = others
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(head)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
