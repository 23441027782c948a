"""Host-side plan rules (fluxbin_plan_of: no device access).

The plan decides only the work division (rows per workgroup, 128-column chunks
per workgroup range, splits); the arithmetic of an output does not depend on it
except through the order of the split combination, which the GPU parity tests
cover.  These tests pin the automatic choices measured on MI355X, so that a
change to the rules shows up here before it shows up as a slower call.
"""
import ctypes

import pytest

from binary_basis_lut_amd import inputs as I


@pytest.fixture(scope="module")
def fb():
    from binary_basis_lut_amd import build as B
    if B.is_stale():
        B.build()
    from binary_basis_lut_amd import fluxbin
    return fluxbin


def desc_for(fb, n, k, kb, ks, s, g=4, **kw):
    d = fb.LayerDesc()
    d.abi_version = fb.ABI_VERSION
    d.g, d.kb, d.ks = g, kb, ks
    d.n, d.k, d.s, d.max_batch = n, k, s, 1
    d.layout = fb.LAYOUT_TILED
    for key, v in kw.items():
        setattr(d, key, v)
    return d


def workload_desc(fb, wid, shape, **kw):
    lay = I.workload_layer(wid, shape, 0)
    return desc_for(fb, lay.n, lay.k, lay.kb, lay.ks, lay.s, g=lay.g, **kw)


def blockwise_desc(fb, n, k, **kw):
    # 2 global + 2 salient bases, 8 salient columns per 128-column group
    return desc_for(fb, n, k, 2, 2, k // 16, row_group=128, sal_group=8, **kw)


def plan(fb, d):
    return fb.fluxbin_plan_of(d)


def test_q_proj_decode_plan(fb):
    # the measured workload: 128 rows per workgroup, four waves per row tile (512 threads), each
    # over 2 chunks of an 8-chunk range: 9 splits over 32 row blocks
    p = plan(fb, workload_desc(fb, 2, 0))
    assert (p["rows_per_block"], p["chunks_per_block"], p["row_blocks"], p["splits"]) == (128, 8, 32, 9)
    assert p["total_chunks"] == 66 and p["grid"] == 288 and p["threads_per_block"] == 512
    # an explicit range length or wave count keeps one wave per row tile
    p = plan(fb, workload_desc(fb, 2, 0, chunks_per_block=2))
    assert (p["rows_per_block"], p["chunks_per_block"], p["threads_per_block"]) == (256, 2, 256)
    p = plan(fb, workload_desc(fb, 2, 0, waves_per_block=4))
    assert (p["rows_per_block"], p["chunks_per_block"], p["threads_per_block"]) == (256, 2, 256)


def test_several_waves_per_row_tile_only_where_ranges_would_be_two_chunks(fb):
    # 7B up 4096 -> 11008 and down 11008 -> 4096 at one batch row take them; the 70B layers
    # (longer ranges or 8-wave workgroups), several batch rows, fp16 entries and block-wise
    # scales do not
    for shape in (0, 1):
        p = plan(fb, workload_desc(fb, 4, shape))
        assert p["threads_per_block"] == 2 * p["rows_per_block"] == 512, shape
        assert p["chunks_per_block"] == 4, shape
    for shape in range(4):
        p = plan(fb, workload_desc(fb, 5, shape))
        assert p["threads_per_block"] == p["rows_per_block"], shape
    assert plan(fb, workload_desc(fb, 4, 0, max_batch=2))["threads_per_block"] == 256
    p = plan(fb, workload_desc(fb, 2, 0, table_precision=fb.TABLE_F16))
    assert p["threads_per_block"] == p["rows_per_block"]
    p = plan(fb, blockwise_desc(fb, 4096, 4096))
    assert p["threads_per_block"] == p["rows_per_block"]
    # nor layers whose one-wave plan has fewer workgroups than the chip has CUs: 512 x 512 keeps
    # 2 x 4 workgroups of 256 threads, 1100 x 4096 its 5 x 33 (a 2100-row layer, 9 x 33, does not)
    p = plan(fb, workload_desc(fb, 1, 0))
    assert (p["grid"], p["threads_per_block"], p["chunks_per_block"]) == (8, 256, 2)
    p = plan(fb, desc_for(fb, 1100, 4096, 2, 1, 100))
    assert (p["grid"], p["threads_per_block"]) == (165, 256)
    p = plan(fb, desc_for(fb, 2100, 4096, 2, 1, 100))
    assert (p["grid"], p["threads_per_block"]) == (153, 512)


def test_four_waves_per_row_tile_where_two_would_be_one_round(fb):
    # four waves per tile where the two-wave grid has at most 512 workgroups and the four-wave one
    # at least 256: q_proj (272 -> 288), 4000 x 4000; the 7B up and down shapes (731, 720
    # workgroups at two) and 2100 x 4096 (153 at four) keep two
    for d, four in ((workload_desc(fb, 2, 0), True), (desc_for(fb, 4000, 4000, 2, 1, 100), True),
                    (workload_desc(fb, 4, 0), False), (workload_desc(fb, 4, 1), False),
                    (desc_for(fb, 2100, 4096, 2, 1, 100), False)):
        p = plan(fb, d)
        assert p["threads_per_block"] == (4 if four else 2) * p["rows_per_block"], (d.n, d.k)
        assert p["chunks_per_block"] <= (8 if four else 4)
    # the LDS holds the partials of the three other waves of each of the two tiles
    p = plan(fb, workload_desc(fb, 2, 0))
    assert p["lds_bytes"] == 8 * (32 * 16 * 4 + 128 * 4) + 256 + 3 * 2 * 64 * 4


def test_tall_layer_takes_eight_waves_and_eight_chunk_ranges(fb):
    # 70B gate+up 8192 -> 57344: 896 row tiles, 8 waves; ranges stop at 8 chunks: each 64-chunk
    # global segment in 8 ranges, the 2 salient chunks in one
    p = plan(fb, workload_desc(fb, 5, 2))
    assert (p["rows_per_block"], p["chunks_per_block"], p["splits"]) == (512, 8, 17)
    p = plan(fb, blockwise_desc(fb, 57344, 8192))
    assert p["rows_per_block"] == 512 and p["chunks_per_block"] == 8


def test_very_wide_single_row_layers_take_eight_waves(fb):
    # 70B down 28672 -> 8192: 128 row tiles x 455 chunks, one batch row, per-row scales: 8 waves,
    # 8-chunk ranges (224 global chunks per basis in 28 ranges, the 7 salient chunks in one),
    # 16 row blocks x 57 ranges
    p = plan(fb, workload_desc(fb, 5, 3))
    assert (p["rows_per_block"], p["chunks_per_block"], p["splits"], p["grid"]) == (512, 8, 57, 912)
    # its block-wise form, and several batch rows, keep 4 waves
    assert plan(fb, blockwise_desc(fb, 8192, 28672))["rows_per_block"] == 256
    assert plan(fb, workload_desc(fb, 5, 3, max_batch=2))["rows_per_block"] == 256
    # qkv and o (160 / 128 row tiles x 130 chunks) stay at 4 waves
    for shape in (0, 1):
        p = plan(fb, workload_desc(fb, 5, shape))
        assert (p["rows_per_block"], p["chunks_per_block"], p["splits"]) == (256, 4, 33)


def test_g8_layers_take_eight_waves_within_the_lds_budget(fb):
    # 7B layer, 3 global bases + 2 % salient, g = 8: 512 rows per workgroup; a chunk's g = 8
    # tables are 16 sub-vectors x 256 entries, 16 KiB per batch row (fp32).  The bank-private layout
    # takes 2-chunk regions (four workgroups per CU): one per range, or two in turn per 4-chunk
    # range where 2-chunk ranges would make more than 1536 workgroups (gate+up: 43 row blocks x 49)
    # or more than 64 ranges (down: 86 chunks per basis)
    expect = {0: (2, 49, 1176), 1: (2, 49, 392), 2: (4, 25, 1075), 3: (4, 67, 536)}
    for shape, (cpb, splits, grid) in expect.items():
        p = plan(fb, workload_desc(fb, 3, shape))
        assert (p["rows_per_block"], p["chunks_per_block"], p["splits"], p["grid"]) == (512, cpb, splits, grid), shape
        # one batch row, per-row scales, fp32 entries: bank-private tables, one 2-chunk region at a time
        assert (p["banked_tables"], p["table_chunks"]) == (2, 2), shape
        assert p["lds_bytes"] == 2 * 16 * 256 * 4 + cpb * 128 * 4, shape
    # a given chunks_per_block of 3 or 4 takes one 4-chunk region, 16 waves (two workgroups per CU)
    p = plan(fb, workload_desc(fb, 3, 3, chunks_per_block=4))
    assert (p["rows_per_block"], p["banked_tables"], p["table_chunks"]) == (1024, 4, 4)
    assert p["lds_bytes"] == 4 * (16 * 256 * 4 + 128 * 4)
    # fp16 entries halve the tables (and keep the one-table-per-sub-vector layout)
    p = plan(fb, workload_desc(fb, 3, 2, table_precision=fb.TABLE_F16, chunks_per_block=4))
    assert p["lds_bytes"] == 4 * (16 * 256 * 2 + 128 * 4) + 256 and p["banked_tables"] == 0
    # a batched g = 8 layer keeps the one-table-per-sub-vector layout, its ranges held whole (two rows
    # of tables for two chunks fill the LDS)
    p = plan(fb, workload_desc(fb, 3, 2, max_batch=2))
    assert (p["chunks_per_block"], p["table_chunks"]) == (2, 2)
    # g = 4 with 8 rows: 4-chunk ranges, tables built two chunks at a time
    p = plan(fb, workload_desc(fb, 4, 0, max_batch=8))
    assert (p["chunks_per_block"], p["table_chunks"]) == (4, 2)
    # so do batched and block-wise g = 8 layers, and every g = 4 layer
    assert plan(fb, workload_desc(fb, 3, 2, max_batch=2))["banked_tables"] == 0
    assert plan(fb, blockwise_desc(fb, 4096, 4096, g=8))["banked_tables"] == 0
    assert plan(fb, workload_desc(fb, 5, 2))["banked_tables"] == 0


def test_explicit_choices_override_the_rules(fb):
    p = plan(fb, workload_desc(fb, 5, 2, waves_per_block=4, chunks_per_block=8))
    assert (p["rows_per_block"], p["chunks_per_block"], p["splits"]) == (256, 8, 17)


def test_range_length_counts_batch_rows(fb):
    # up 4096 -> 11008: 2 chunks per wave at one batch row (two waves over each 4-chunk range),
    # 4 at two and four (a group of nb rows counts nb times); the LDS caps four-row ranges at 4
    p = plan(fb, workload_desc(fb, 4, 0))
    assert p["chunks_per_block"] == 4 and p["threads_per_block"] == 2 * p["rows_per_block"]
    assert plan(fb, workload_desc(fb, 4, 0, max_batch=2))["chunks_per_block"] == 4
    p = plan(fb, workload_desc(fb, 4, 0, max_batch=4))
    assert p["chunks_per_block"] == 4 and p["splits"] == 17
    # q_proj stays at 2 chunks for two batch rows
    assert plan(fb, workload_desc(fb, 2, 0, max_batch=2))["chunks_per_block"] == 2


def test_plan_of_rejects_like_workspace_size(fb):
    info = fb.PlanInfo()
    bad = workload_desc(fb, 2, 0)
    bad.kb = 5  # supported: 1..4
    assert fb.raw_status("fluxbin_plan_of", ctypes.byref(bad), ctypes.byref(info)) == fb.ERR_UNSUPPORTED
    out = ctypes.c_size_t(0)
    assert fb.raw_status("fluxbin_workspace_size", ctypes.byref(bad), ctypes.byref(out)) == fb.ERR_UNSUPPORTED
    good = workload_desc(fb, 2, 0)
    assert fb.raw_status("fluxbin_plan_of", ctypes.byref(good), None) == fb.ERR_INVALID_ARGUMENT
    assert fb.raw_status("fluxbin_plan_of", None, ctypes.byref(info)) == fb.ERR_INVALID_ARGUMENT


@pytest.mark.gpu
def test_plan_of_matches_the_handle(fb):
    # the host-side query and a created handle agree (one, four and 64 batch rows)
    for lay, kw in [(I.workload_layer(2, 0, 0), {}), (I.workload_layer(4, 1, 0), {"max_batch": 4}),
                    (I.workload_layer(4, 0, 0), {"max_batch": 64})]:
        dl = fb.DeviceLayer(lay, kw.get("max_batch", 1))
        d = desc_for(fb, lay.n, lay.k, lay.kb, lay.ks, lay.s, g=lay.g, **kw)
        assert fb.fluxbin_plan_of(d) == dl.plan, (lay.n, lay.k, kw)
        dl.close()
