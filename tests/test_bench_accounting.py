"""bench.py's byte/flop accounting against the pages' printed numbers.

tests/golden/gqa_cache_counts.json: the GQA cache-size example of
"注意力优化（Attention Optimization）" (262144 vs 65536 entries, 75% saved) and
the decode equations 5-6 of the NVIDIA co-design blog.
"""
import json
import os

import bench


def test_gqa_example_counts(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "gqa_cache_counts.json")))["gqa_example"]
    mha = bench.gqa_cache_elements(g["heads"], g["head_dim"], g["seq_len"])
    gqa = bench.gqa_cache_elements(g["kv_heads"], g["head_dim"], g["seq_len"])
    assert mha == g["mha"] and gqa == g["gqa"]
    assert round((1 - gqa / mha) * 100) == g["saving_percent"]


def test_decode_equations(golden_dir):
    for case in json.load(open(os.path.join(golden_dir, "gqa_cache_counts.json")))["decode_eq"]:
        qh = case["KH"] * case["G"]
        assert bench.decode_eq_flops(case["DB"], qh, case["KVSL"], case["Hsz"]) == case["flops"]
        assert bench.decode_eq_elements(case["DB"], case["KH"], case["G"], case["Hsz"], case["KVSL"]) == case["elements"]
        # the KV part of equation 6 is what the bench counts as KV bytes (2 bytes per bf16 element)
        kv = bench.kv_bytes(case["DB"] * case["KVSL"], case["KH"], case["Hsz"], 2)
        qo = 2 * case["DB"] * case["KH"] * case["Hsz"] * case["G"] * 2
        assert kv + qo == case["elements"] * 2


def test_partial_bytes():
    # one (m, l, o[D]) fp32 triple per (row, chunk)
    assert bench.partial_bytes(1, 128) == 130 * 4
