"""Device-side helpers for the GPU parity tests (data movement only)."""
import math

import numpy as np
import torch

import long_context_decode_gqa_amd as pkg
import oracle
import synth

DEV = torch.device("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    """Host array -> device tensor; uint16 arrays are bf16 bit patterns."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def dev_geom(g: synth.Geometry) -> pkg.KVGeometry:
    return pkg.KVGeometry(g.B, g.KH, g.D, int(g.max_len) if g.B else 0, torch.from_numpy(g.lens).to(DEV),
                          torch.from_numpy(g.seq_offset).to(DEV), g.stride_h, g.stride_t)


def problem(w, q, k, v, g, **kw):
    return oracle.Problem(w.B, w.KH, w.G, w.D, g.lens, g.seq_offset, g.stride_h, g.stride_t,
                          np.ascontiguousarray(q), k, v, 1.0 / math.sqrt(w.D), **kw)


def bf16_to_f32(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


def log_case(msg: str):
    print(f"[case] {msg}", flush=True)


def host_threads() -> int:
    """Host threads for the oracle: the cores this process may use, capped by the CPU share the
    machine grants it (OMP_NUM_THREADS where set)."""
    import os
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    share = os.environ.get("OMP_NUM_THREADS", "")
    if share.isdigit() and int(share) > 0:
        n = min(n, int(share))
    return max(1, n)


def oracle_all_rows(p):
    """The oracle over every output row of a problem, on all host threads; logs the host time."""
    import time
    t0 = time.perf_counter()
    ref, ref_lse = oracle.attention_rows(p, oracle.all_rows(p), nthreads=host_threads())
    print(f"[info] oracle over {ref.shape[0]} rows: {time.perf_counter() - t0:.1f} s on {host_threads()} threads",
          flush=True)
    return ref, ref_lse
