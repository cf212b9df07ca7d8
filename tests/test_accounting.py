"""The byte/FLOP model used for `achieved` bandwidth, pinned to figures the
pages print (tests/golden/pages_accounting.json) and to direct counts."""

import json
import os

import numpy as np
import pytest

from decode_attention_mfa_amd import accounting as acc

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_accounting.json")))


def rel(a, b):
    return abs(a - b) / abs(b)


@pytest.mark.parametrize("key", ["step3_table2_8k", "step3_table3_32k"])
def test_step3_per_token_tables(key):
    g = GOLD[key]
    kv, fl = acc.per_token_model(g["layers"], g["context"], hq=64, hkv=1, d=256, kv_bytes=1)
    assert rel(kv, g["kv_bytes"]) < 5e-3
    assert rel(fl, g["attention_flops"]) < 5e-3


def test_step3_intensity_and_bytes_per_token():
    per_key_bytes = acc.kv_bytes_per_token(1, 256, 1)
    assert per_key_bytes == GOLD["step3_kv_bytes_per_token"]["value"]
    assert acc.attention_flops_per_key(64, 256) / per_key_bytes == \
        GOLD["step3_intensity_8bit"]["value"]


def test_step5_cache_formula():
    assert acc.kv_bytes_per_token(4, 192, 2) == GOLD["step5_kv_bytes_per_token_layer"]["value"]
    g = GOLD["step5_payload_1m"]
    glob, loc, summ = acc.step5_cache_payload(g["T"])
    assert acc.gib(glob) == pytest.approx(g["global_gib"], rel=1e-9)
    assert acc.mib(loc) == pytest.approx(g["local_mib"], rel=1e-9)
    assert acc.mib(summ) == pytest.approx(g["summary_mib"], rel=1e-9)
    assert acc.gib(glob + loc + summ) == pytest.approx(g["total_gib"], rel=1e-7)


def test_headline_call_bytes():
    lens = np.full(64, 4096)
    b = acc.decode_call_bytes(lens, hq=64, hkv=1, d=256, q_fmt="bf16", kv_fmt="bf16",
                              out_fmt="bf16")
    kv = 64 * 4096 * 256 * 2 * 2
    assert b == kv + 64 * 64 * 256 * 4 + 64 * (4 * 64 + 4)
    assert round(b / 1e6, 1) == 272.6
    assert acc.decode_call_flops(lens, hq=64, d=256) == 64 * 4096 * 65536


def test_window_counts_only_attended_keys_and_touched_pages():
    assert acc.attended_keys(32768, 512) == 512
    assert acc.pages_touched(32768, 512) == 8          # aligned window
    assert acc.pages_touched(32769, 512) == 9          # straddles a page
    assert acc.pages_touched(100, 512) == 2
    assert acc.pages_touched(0) == 0


def test_query_path_work_against_the_linear_column():
    # Table 2's linear column counts every projection of a layer per token; the
    # query path (two products, 7168 -> 2048 -> 64 x 256) is most of it.  With
    # the K, V and output projections of Table 1's shape added back it must
    # reproduce the printed figure, and at batch 256 the path moves the bf16
    # weights once plus x and q.
    g = GOLD["step3_table2_linear_8k"]
    q_bytes, q_flops = acc.query_proj_work(1)
    kv_o_flops = 2 * (2 * 7168 * 256 + 64 * 256 * 7168)
    total = g["layers"] * (q_flops + kv_o_flops)
    assert abs(total - g["linear_flops"]) / g["linear_flops"] < 0.005
    nbytes, flops = acc.query_proj_work(256)
    assert flops == 2 * 256 * (7168 * 2048 + 2048 * 16384)
    assert nbytes == 2 * (7168 * 2048 + 2048 * 16384) + 2 * 256 * (7168 + 16384)
