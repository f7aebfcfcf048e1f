"""The C ABI library loads, exports every declared entry point, and rejects bad
arguments on the host before touching a GPU (no compute calls here)."""
import ctypes
import os
import re

import pytest

import long_context_decode_gqa_amd as pkg
from long_context_decode_gqa_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_decode.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^(?:const\s+)?(?:attn_status|char|size_t|void|int32_t)\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_four_method_calls():
    names = declared_functions()
    for n in ("attn_decode_splitkv", "attn_merge_lse", "kv_quant_int8", "oam_score_topk"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = _lib.load()
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib.SIGNATURES), "binding signatures out of sync with the header"


def test_status_strings():
    L = _lib.load()
    assert L.attn_status_string(0) == b"ok"
    assert L.attn_status_string(3) == b"workspace too small"


FAKE = 0x10000  # never dereferenced: validation fails or only sizes are computed


def _args(**over):
    a = _lib.AttnDecodeArgs()
    a.kv = _lib.AttnKvGeom(2, 8, 128, 4096, FAKE, FAKE, 4096 * 128, 128)
    a.G = 8
    a.q_dtype = a.kv_dtype = _lib.ATTN_BF16
    a.out_dtype = _lib.ATTN_F32
    a.q = a.k = a.v = a.out = FAKE
    for k, v in over.items():
        if k.startswith("g_"):
            setattr(a.kv, k[2:], v)
        else:
            setattr(a, k, v)
    return a


def _ws(a):
    n = ctypes.c_size_t(0)
    st = _lib.load().attn_decode_workspace_size(ctypes.byref(a), ctypes.byref(n))
    return st, n.value


def test_workspace_size_counts_partials():
    st, n = _ws(_args(split_tokens=1024))
    assert st == 0
    partials = 2 * 64 * 4   # B * QH * ceil(4096 / 1024)
    assert n >= partials * (128 + 2) * 4
    st2, n2 = _ws(_args(split_tokens=512))
    assert st2 == 0 and n2 > n


def _split(a):
    n = ctypes.c_int32(0)
    st = _lib.load().attn_decode_split_tokens(ctypes.byref(a), ctypes.byref(n))
    return st, n.value


I8 = dict(kv_dtype=_lib.ATTN_I8, k_scale=FAKE, k_part_tokens=64, k_scale_stride=2048)


@pytest.mark.parametrize("over,split", [
    # bf16 and int8 KV: workers of four waves, each wave streaming at least 32 tiles of 32
    # positions, so a worker's range is at least 4096 positions (the grid's size decides the rest)
    (dict(g_B=4, g_max_seq_len=131072), 4096),
    (dict(g_B=4, g_max_seq_len=131072, **I8), 4096),
    (dict(g_B=4, g_max_seq_len=131072, q_rows=4), 4096),
    (dict(g_B=4, g_KH=1, g_max_seq_len=131072), 4096),
    (dict(g_B=1, g_KH=1, g_max_seq_len=4096), 4096),
    (dict(g_B=4, g_max_seq_len=131072, g_seq_offset=None, g_block_table=FAKE, g_page_tokens=32,
          g_table_stride=4096, g_page_stride=32 * 8 * 128, **I8), 4096),
    # token-major pages (a KV head's rows KH * D apart): twice the workers over half the range
    (dict(g_B=4, g_max_seq_len=131072, g_seq_offset=None, g_block_table=FAKE, g_page_tokens=64,
          g_table_stride=2048, g_page_stride=64 * 8 * 128, g_stride_h=128, g_stride_t=8 * 128), 2048),
    # a contiguous token-major cache keeps the one-round split
    (dict(g_B=4, g_max_seq_len=131072, g_stride_h=128, g_stride_t=8 * 128), 4096),
    # kept-token lists: at least 512 and at most 1024 kept tokens per worker
    (dict(g_B=4, g_max_seq_len=131072, token_idx=FAKE, n_idx=FAKE, idx_stride=4096), 512),
    (dict(g_B=4, g_max_seq_len=131072, token_idx=FAKE, n_idx=FAKE, idx_stride=4096, **I8), 512),
    (dict(g_B=4, g_max_seq_len=131072, token_idx=FAKE, n_idx=FAKE, idx_stride=16384), 1024),
    # fp32 KV (vector-ALU decode): chunks of 256
    (dict(q_dtype=_lib.ATTN_F32, kv_dtype=_lib.ATTN_F32), 256),
    # a given split is kept
    (dict(split_tokens=96), 96),
])
def test_default_split_tokens(over, split):
    """The library's default split_tokens, as attn_decode_split_tokens reports it: the smallest
    range of positions a decode worker takes (workers = min(grid, positions / split_tokens))."""
    st, n = _split(_args(**over))
    assert st == 0 and n == split, (over, n)
    assert _split(_args(G=0))[0] == _lib.ATTN_ERR_UNSUPPORTED


@pytest.mark.parametrize("over,status", [
    (dict(G=0), _lib.ATTN_ERR_UNSUPPORTED),
    (dict(G=65), _lib.ATTN_ERR_UNSUPPORTED),
    (dict(g_D=96), _lib.ATTN_ERR_UNSUPPORTED),
    (dict(g_KH=0), _lib.ATTN_ERR_INVALID_ARG),
    (dict(g_B=-1), _lib.ATTN_ERR_INVALID_ARG),
    (dict(g_stride_t=100), _lib.ATTN_ERR_INVALID_ARG),
    (dict(g_stride_t=132), _lib.ATTN_ERR_INVALID_ARG),
    (dict(q_dtype=_lib.ATTN_F32), _lib.ATTN_ERR_UNSUPPORTED),
    (dict(kv_dtype=7), _lib.ATTN_ERR_INVALID_ARG),
    (dict(out_dtype=_lib.ATTN_I8), _lib.ATTN_ERR_INVALID_ARG),
    (dict(split_tokens=48), _lib.ATTN_ERR_INVALID_ARG),
    (dict(q=None), _lib.ATTN_ERR_INVALID_ARG),
    (dict(k=FAKE + 8), _lib.ATTN_ERR_INVALID_ARG),
    (dict(g_seq_lens=None), _lib.ATTN_ERR_INVALID_ARG),
    (dict(kv_dtype=_lib.ATTN_I8), _lib.ATTN_ERR_INVALID_ARG),          # no k_scale
    (dict(kv_dtype=_lib.ATTN_I8, k_scale=FAKE, k_part_tokens=64, k_scale_stride=3), _lib.ATTN_ERR_INVALID_ARG),
    (dict(kv_dtype=_lib.ATTN_I8, k_scale=FAKE, k_part_tokens=40, k_scale_stride=64), _lib.ATTN_ERR_INVALID_ARG),
    (dict(token_idx=FAKE), _lib.ATTN_ERR_INVALID_ARG),                 # no n_idx
    (dict(fixed_splits=-1), _lib.ATTN_ERR_INVALID_ARG),
    (dict(fixed_splits=70000), _lib.ATTN_ERR_INVALID_ARG),
    (dict(fixed_splits=2, q_dtype=_lib.ATTN_F32, kv_dtype=_lib.ATTN_F32), _lib.ATTN_ERR_UNSUPPORTED),
    (dict(softmax_scale=float("inf")), _lib.ATTN_ERR_INVALID_ARG),
    (dict(q_quant=3), _lib.ATTN_ERR_INVALID_ARG),
    (dict(q_quant=_lib.ATTN_QUANT_ROW), _lib.ATTN_ERR_UNSUPPORTED),   # int8 query needs int8 KV
    (dict(kv_dtype=_lib.ATTN_I8, k_scale=FAKE, k_part_tokens=0, q_quant=_lib.ATTN_QUANT_STATIC, q_scale=-1.0),
     _lib.ATTN_ERR_INVALID_ARG),
    (dict(kv_dtype=_lib.ATTN_I8, k_scale=FAKE, k_part_tokens=0, q_quant=_lib.ATTN_QUANT_STATIC,
          q_scale=float("inf")), _lib.ATTN_ERR_INVALID_ARG),
    (dict(kv_dtype=_lib.ATTN_I8, k_scale=FAKE, k_part_tokens=-64, k_scale_stride=64), _lib.ATTN_ERR_INVALID_ARG),
])
def test_invalid_arguments_are_rejected_on_the_host(over, status):
    a = _args(**over)
    st, _ = _ws(a)
    assert st == status
    # the enqueueing call fails the same way, before any HIP call
    assert _lib.load().attn_decode_splitkv(ctypes.byref(a), None) == status
    assert _lib.load().attn_last_error()


def test_workspace_too_small_is_reported_before_launch():
    a = _args(workspace=0x100000, workspace_bytes=1024)
    assert _lib.load().attn_decode_splitkv(ctypes.byref(a), None) == _lib.ATTN_ERR_WORKSPACE_TOO_SMALL
    a = _args(workspace=0x100010, workspace_bytes=1 << 30)
    assert _lib.load().attn_decode_splitkv(ctypes.byref(a), None) == _lib.ATTN_ERR_INVALID_ARG  # misaligned


def test_int8_and_fp32_paths_validate():
    assert _ws(_args(kv_dtype=_lib.ATTN_I8, k_scale=FAKE, k_part_tokens=64, k_scale_stride=64))[0] == 0
    # per-tensor K (k_part_tokens 0, stride ignored) with each query mode
    for qq, qs in ((_lib.ATTN_QUANT_EXACT, 0.0), (_lib.ATTN_QUANT_ROW, 0.0), (_lib.ATTN_QUANT_STATIC, 0.02)):
        assert _ws(_args(kv_dtype=_lib.ATTN_I8, k_scale=FAKE, k_part_tokens=0, q_quant=qq, q_scale=qs))[0] == 0
    a = _args(q_dtype=_lib.ATTN_F32, kv_dtype=_lib.ATTN_F32, g_D=64, g_stride_h=4096 * 64, g_stride_t=64)
    assert _ws(a)[0] == 0
    a = _args(q_dtype=_lib.ATTN_F32, kv_dtype=_lib.ATTN_F32, g_D=66, g_stride_h=4096 * 68, g_stride_t=68)
    assert _ws(a)[0] == _lib.ATTN_ERR_UNSUPPORTED


def test_merge_and_quant_validation():
    L = _lib.load()
    assert L.attn_merge_lse(None, None, None, None, 0, 128, 0, None, None, None) == 0
    assert L.attn_merge_lse(FAKE, FAKE, FAKE, None, 4, 128, 0, FAKE, None, None) == _lib.ATTN_ERR_INVALID_ARG
    assert L.attn_merge_lse(FAKE, FAKE, FAKE, FAKE, 4, 300, 0, FAKE, None, None) == _lib.ATTN_ERR_UNSUPPORTED
    g = _lib.AttnKvGeom(2, 8, 128, 4096, FAKE, FAKE, 4096 * 128, 128)
    assert L.kv_quant_int8(ctypes.byref(g), FAKE, 40, 200, FAKE, FAKE, None, 0, None) == _lib.ATTN_ERR_INVALID_ARG
    assert L.kv_quant_int8(ctypes.byref(g), FAKE, 64, 10, FAKE, FAKE, None, 0, None) == _lib.ATTN_ERR_INVALID_ARG
    assert L.kv_quant_int8(ctypes.byref(g), FAKE, 0, 1, FAKE, FAKE, None, 0, None) == \
        _lib.ATTN_ERR_WORKSPACE_TOO_SMALL
    n = ctypes.c_size_t(7)
    assert L.kv_quant_int8_workspace_size(ctypes.byref(g), 0, ctypes.byref(n)) == 0
    # per-tensor mode: 256 bytes + one float per four 64-row blocks (D = 128) per (b, kh):
    # 4096 rows -> 64 blocks -> 16 groups, x 2 sequences x 8 KV heads
    assert n.value == 256 + 4 * 16 * 2 * 8
    assert L.kv_quant_int8(ctypes.byref(g), FAKE, 0, 1, FAKE, FAKE, FAKE, n.value - 4, None) == \
        _lib.ATTN_ERR_WORKSPACE_TOO_SMALL
    assert L.kv_quant_int8_workspace_size(ctypes.byref(g), 64, ctypes.byref(n)) == 0 and n.value == 0


def test_argument_structs_match_the_header_layout(tmp_path):
    """The binding's ctypes structs have the C header's field offsets and sizes (gcc on this host)."""
    structs = {"attn_decode_args": _lib.AttnDecodeArgs, "attn_kv_geom": _lib.AttnKvGeom,
               "oam_topk_args": _lib.OamTopkArgs}
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "attn_decode.h"', "int main(void) {"]
    for cname, cls in structs.items():
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for f in cls._fields_:
            lines.append(f'printf("{cname} {f[0]} %zu\\n", offsetof({cname}, {f[0]}));')
    lines += ["return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    import subprocess
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {tuple(l.split()[:2]): int(l.split()[2]) for l in out if l}
    for cname, cls in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(cls), cname
        for f in cls._fields_:
            assert got[(cname, f[0])] == getattr(cls, f[0]).offset, (cname, f[0])


def test_paged_geometry_is_validated():
    L = _lib.load()
    paged = dict(g_block_table=FAKE, g_page_tokens=64, g_table_stride=64, g_page_stride=64 * 8 * 128,
                 g_seq_offset=None)
    assert _ws(_args(**paged))[0] == 0
    assert _ws(_args(**paged, kv_dtype=_lib.ATTN_I8, k_scale=FAKE, k_part_tokens=64, k_scale_stride=64))[0] == 0
    for over, status in ((dict(g_page_tokens=48), _lib.ATTN_ERR_INVALID_ARG),
                         (dict(g_table_stride=63), _lib.ATTN_ERR_INVALID_ARG),
                         (dict(g_page_stride=0), _lib.ATTN_ERR_INVALID_ARG),
                         (dict(g_page_tokens=32, split_tokens=1 << 20), _lib.ATTN_OK),
                         (dict(token_idx=FAKE, n_idx=FAKE, idx_stride=10), _lib.ATTN_ERR_UNSUPPORTED),
                         (dict(q_dtype=_lib.ATTN_F32, kv_dtype=_lib.ATTN_F32), _lib.ATTN_ERR_UNSUPPORTED)):
        a = _args(**{**paged, **over})
        if "g_page_tokens" in over and over["g_page_tokens"] == 32:
            a.kv.table_stride = 128  # 4096 tokens in 32-token pages
        assert _ws(a)[0] == status, over
    # the quantiser, the value norms and OAM selection read a paged cache too; their geometry
    # checks still run before any launch (a page stride of 4 bf16 elements is not 16-byte aligned)
    g = _lib.AttnKvGeom(2, 8, 128, 4096, FAKE, None, 128, 1024)
    g.block_table, g.page_tokens, g.table_stride, g.page_stride = FAKE, 64, 64, 64 * 1024 + 4
    assert L.kv_quant_int8(ctypes.byref(g), FAKE, 64, 64, FAKE, FAKE, None, 0, None) == _lib.ATTN_ERR_INVALID_ARG
    vlog = ctypes.c_void_p(FAKE)
    assert L.oam_value_lognorm(ctypes.byref(g), FAKE, _lib.ATTN_BF16, 1.0, 1e-6, vlog, 4096, None) == \
        _lib.ATTN_ERR_INVALID_ARG
    n = ctypes.c_size_t(0)
    assert L.kv_quant_int8_workspace_size(ctypes.byref(g), 0, ctypes.byref(n)) == _lib.ATTN_ERR_INVALID_ARG
    g.page_stride = 64 * 1024
    assert L.kv_quant_int8_workspace_size(ctypes.byref(g), 0, ctypes.byref(n)) == 0 and n.value > 256
    o = _lib.OamTopkArgs()
    o.kv, o.G, o.q, o.k, o.kv_dtype, o.vlog, o.vlog_stride = g, 8, FAKE, FAKE, _lib.ATTN_BF16, FAKE, 4096
    o.top_k, o.idx_out, o.n_kept, o.beta, o.eps = 512, FAKE, FAKE, 1.0, 1e-6
    assert L.oam_score_topk_workspace_size(ctypes.byref(o), ctypes.byref(n)) == 0 and n.value > 0
    o.kv.page_stride = 64 * 1024 + 4
    assert L.oam_score_topk_workspace_size(ctypes.byref(o), ctypes.byref(n)) == _lib.ATTN_ERR_INVALID_ARG


def test_long_paged_token_major_cache_is_accepted():
    """A paged cache's buffer offsets span one page, not one sequence: a token-major pool
    (KH=8, D=128 bf16, 2 KiB per token row) of 1.5M-token sequences is accepted by the decode and
    OAM workspace queries, while the same length in one contiguous (sequence, head) is not."""
    L = _lib.load()
    n_tok = 3 << 19
    pages = n_tok // 64
    paged = dict(g_B=2, g_max_seq_len=n_tok, g_block_table=FAKE, g_page_tokens=64, g_table_stride=pages,
                 g_page_stride=64 * 8 * 128, g_seq_offset=None, g_stride_h=128, g_stride_t=8 * 128)
    assert _ws(_args(**paged))[0] == _lib.ATTN_OK
    contiguous = dict(g_B=2, g_max_seq_len=n_tok, g_stride_h=128, g_stride_t=8 * 128)
    assert _ws(_args(**contiguous))[0] == _lib.ATTN_ERR_UNSUPPORTED
    g = _lib.AttnKvGeom(2, 8, 128, n_tok, FAKE, None, 128, 8 * 128)
    g.block_table, g.page_tokens, g.table_stride, g.page_stride = FAKE, 64, pages, 64 * 8 * 128
    o = _lib.OamTopkArgs()
    o.kv, o.G, o.q, o.k, o.kv_dtype, o.vlog, o.vlog_stride = g, 8, FAKE, FAKE, _lib.ATTN_BF16, FAKE, n_tok
    o.top_k, o.idx_out, o.n_kept, o.beta, o.eps = 4096, FAKE, FAKE, 1.0, 1e-6
    n = ctypes.c_size_t(0)
    assert L.oam_score_topk_workspace_size(ctypes.byref(o), ctypes.byref(n)) == _lib.ATTN_OK
