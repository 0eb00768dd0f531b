"""The offline key-table sweeper's selection logic and the compiled table
(host only; the measuring half runs on a GPU)."""
import os

import pytest

from deterministic_persistent_gemm_amd import sweep

bi = pytest.importorskip("deterministic_persistent_gemm_amd")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def cand(bk, dec, per):
    return {"block_k": bk, "decode": dec, "persistent": per}


def test_summary_crossover_and_tiles():
    c = cand(128,
             {1: {1: 10.0, 3: 12.0}, 8: {1: 10.5, 3: 11.0}, 64: {1: 13.0}, 128: {1: 16.0}},
             {1: {4: 40.0}, 8: {4: 40.0}, 64: {4: 20.0, 3: 14.0}, 128: {3: 15.0, 4: 15.5},
              256: {3: 20.0}, 1024: {3: 45.0, 4: 50.0}, 4096: {4: 97.0, 3: 120.0}})
    s = sweep.summarize(c)
    # the persistent kernel wins from M=128 on; decode serves up to 64
    assert s["m_decode_max"] == 64 and s["decode_path"] == 1
    # 32x32 (code 3) up to 1024, 64x64 (code 4) above
    assert (s["m_a"], s["tile_a"], s["tile_c"]) == (1024, 3, 4)
    assert s["decode_total_us"] == 10.0 + 10.5 + 13.0 + 15.0
    assert s["prefill_total_us"] == 20.0 + 45.0 + 97.0


def test_profiles_pick_the_trade_off():
    a = {"block_k": 128, "decode_total_us": 50.0, "prefill_total_us": 200.0}
    b = {"block_k": 512, "decode_total_us": 60.0, "prefill_total_us": 150.0}
    assert sweep.choose([a, b], "decode")["block_k"] == 128
    assert sweep.choose([a, b], "prefill")["block_k"] == 512
    # balanced: 50/50 + 200/150 = 2.33 against 60/50 + 1 = 2.2
    assert sweep.choose([a, b], "balanced")["block_k"] == 512
    # within the tie band the served recipe stays
    c = {"block_k": 256, "decode_total_us": 49.0, "prefill_total_us": 210.0}
    assert sweep.choose([a, c], "decode", keep_block_k=128, tie=0.03)["block_k"] == 128
    assert sweep.choose([a, c], "decode", keep_block_k=128, tie=0.0)["block_k"] == 256


def test_tile_codes_skip_shapes_that_fall_back():
    assert sweep.tile_codes("f32", 4096, 128) == tuple(range(1, 11)) + (23, 24, 28, 29)
    # 128-k stages (9, 10) do not divide 320; the rings (23, 24) need several k tiles
    assert sweep.tile_codes("f32", 320, 320) == (1, 2, 3, 4, 5, 6, 7, 8)
    assert 18 not in sweep.tile_codes("bf16", 4096, 512)        # 256x256 needs one k tile
    assert {18, 19} <= set(sweep.tile_codes("bf16", 4096, 4096))
    assert sweep.parse_key("bf16:4096:4096:balanced") == ("bf16", 4096, 4096, "balanced")
    assert sweep.parse_key("f32:256:4096") == ("f32", 256, 4096, "decode")


def test_tile_ranges_merge_to_three():
    per = {128: {12: 20.0, 13: 30.0, 16: 22.0}, 256: {12: 32.0, 13: 58.0, 16: 39.0},
           512: {12: 40.0, 13: 45.0, 16: 41.0}, 1024: {12: 74.0, 13: 64.0, 16: 85.0},
           4096: {12: 275.0, 13: 233.0, 19: 127.0}}
    t = sweep.tile_segments(per, [128, 256, 512, 1024, 4096])
    assert t == {"m_a": 512, "tile_a": 12, "m_b": 1024, "tile_b": 13, "tile_c": 19}
    # four ranges: the cheapest neighbouring pair is merged
    per2 = {1: {1: 1.0, 2: 1.1}, 2: {1: 2.0, 2: 1.0}, 3: {1: 1.0, 2: 3.0}, 4: {1: 5.0, 2: 1.0}}
    t2 = sweep.tile_segments(per2, [1, 2, 3, 4])
    assert t2 == {"m_a": 2, "tile_a": 2, "m_b": 3, "tile_b": 1, "tile_c": 2}


def test_table_lines_merge_and_parse():
    e = {"block_k": 128, "m_decode_max": 128, "decode_path": 1, "m_a": 1024, "tile_a": 3, "m_b": 1024,
         "tile_b": 4, "tile_c": 4, "m_xcd_max": 64}
    line = sweep.table_line("f32", 256, 4096, e)
    assert line == "{BI_F32, 256, 4096, 128, 128, 1, 1024, 3, 1024, 4, 4, 64},"
    assert sweep.parse_table(line)[0]["m_xcd_max"] == 64
    text = sweep.merge_table(sweep.TABLE_HEADER, {"BI_F32,256,4096": line})
    e2 = dict(e, block_k=256)
    text = sweep.merge_table(text, {"BI_F32,256,4096": sweep.table_line("f32", 256, 4096, e2),
                                    "BI_BF16,4096,4096": sweep.table_line("bf16", 4096, 4096, e)})
    rows = sweep.parse_table(text)
    assert [(r["dtype"], r["N"], r["K"], r["block_k"]) for r in rows] == [
        ("BI_F32", 256, 4096, 256), ("BI_BF16", 4096, 4096, 128)]
    assert text.startswith("// Measured key table")


def test_block_k_candidates():
    assert sweep.block_k_candidates("f32", 4096) == [128, 256, 512, 4096]
    assert sweep.block_k_candidates("f32", 320) == [320]
    assert sweep.block_k_candidates("bf16", 768) == [768]
    assert sweep.block_k_candidates("bf16", 2048) == [512, 1024, 2048]


def test_compiled_table_is_what_the_library_serves():
    # every entry of the committed table is a valid recipe the library reports
    # for its key, with tile codes of its dtype
    rows = sweep.parse_table(open(sweep.TABLE).read())
    for r in rows:
        dt = bi.BI_F32 if r["dtype"] == "BI_F32" else bi.BI_BF16
        rec = bi.bi_describe_recipe(dt, r["N"], r["K"])
        assert rec.block_k == r["block_k"], r
        assert rec.m_decode_max == r["m_decode_max"], r
        assert r["K"] % r["block_k"] == 0 and r["block_k"] % 32 == 0
        codes = (*range(1, 11), 23, 24, 28, 29) if dt == bi.BI_F32 else range(11, 23)
        for t in (r["tile_a"], r["tile_b"], r["tile_c"]):
            assert t == 0 or t in codes, r
        assert r["decode_path"] in (0, 1, 3, 4)
        # the XCD hand-over serves a prefix of the decode range, and only keys
        # whose N tiles split evenly over the eight XCDs
        assert 0 <= r["m_xcd_max"] <= r["m_decode_max"], r
        assert r["m_xcd_max"] == 0 or (r["N"] // 16) % 8 == 0, r
        if r["m_xcd_max"]:
            assert bi.plan_path(dt, 1, r["N"], r["K"]) == bi.BI_PATH_DECODE_XCD, r


def test_summary_xcd_prefix_and_other_decode_form():
    # the XCD hand-over (5) is best up to M=32, the two-launch decode (1)
    # from 64; decode_path is picked among the non-XCD forms
    c = cand(128,
             {1: {1: 6.7, 5: 5.6, 3: 13.0}, 8: {1: 7.0, 5: 5.8}, 32: {1: 8.0, 5: 6.7}, 64: {1: 9.4, 5: 9.8},
              128: {1: 12.8, 5: 13.3}},
             {1: {3: 40.0}, 8: {3: 40.0}, 32: {3: 40.0}, 64: {3: 30.0}, 128: {3: 31.0}, 4096: {10: 90.0}})
    s = sweep.summarize(c)
    assert s["m_xcd_max"] == 32 and s["decode_path"] == 1 and s["m_decode_max"] == 128
    # a hand-over that loses at the first point serves nothing
    c["decode"][1][5] = 7.0
    assert sweep.summarize(c)["m_xcd_max"] == 0
