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
    # the measured workload: 4 waves (256 rows), 2-chunk ranges, 33 splits over 16 row blocks
    p = plan(fb, workload_desc(fb, 2, 0))
    assert (p["rows_per_block"], p["chunks_per_block"], p["row_blocks"], p["splits"]) == (256, 2, 16, 33)
    assert p["total_chunks"] == 66 and p["grid"] == 528


def test_tall_layer_takes_eight_waves_and_seven_chunk_ranges(fb):
    # 70B gate+up 8192 -> 57344: 896 row tiles, 8 waves; g = 4 eight-wave ranges stop at 7 chunks
    p = plan(fb, workload_desc(fb, 5, 2))
    assert (p["rows_per_block"], p["chunks_per_block"], p["splits"]) == (512, 7, 19)
    p = plan(fb, blockwise_desc(fb, 57344, 8192))
    assert p["rows_per_block"] == 512 and p["chunks_per_block"] == 7


def test_large_per_row_layer_takes_eight_waves(fb):
    # 70B down 28672 -> 8192: 128 row tiles x 455 chunks of per-row work: 8 waves
    p = plan(fb, workload_desc(fb, 5, 3))
    assert (p["rows_per_block"], p["chunks_per_block"], p["splits"]) == (512, 4, 114)
    # the same shape with block-wise scales keeps 4 waves
    assert plan(fb, blockwise_desc(fb, 8192, 28672))["rows_per_block"] == 256
    # qkv and o (160 / 128 row tiles x 130 chunks) stay at 4 waves
    for shape in (0, 1):
        p = plan(fb, workload_desc(fb, 5, shape))
        assert (p["rows_per_block"], p["chunks_per_block"], p["splits"]) == (256, 4, 33)


def test_g8_layers_take_eight_waves_within_the_lds_budget(fb):
    # 7B layer, 3 global bases + 2 % salient, g = 8: 512 rows per workgroup; a chunk's g = 8
    # tables are 16 sub-vectors x 256 entries, 16 KiB per batch row (fp32), so qkv and down take
    # 2-chunk ranges and the gate+up projection 4 (64 KiB of tables plus the staged inputs)
    expect = {0: (2, 49), 1: (2, 49), 2: (4, 25), 3: (2, 130)}
    for shape, (cpb, splits) in expect.items():
        p = plan(fb, workload_desc(fb, 3, shape))
        assert (p["rows_per_block"], p["chunks_per_block"], p["splits"]) == (512, cpb, splits), shape
    assert plan(fb, workload_desc(fb, 3, 2))["lds_bytes"] == 4 * (16 * 256 * 4 + 128 * 4) + 256
    # fp16 entries halve the tables
    assert plan(fb, workload_desc(fb, 3, 2, table_precision=fb.TABLE_F16, chunks_per_block=4))["lds_bytes"] == \
        4 * (16 * 256 * 2 + 128 * 4) + 256


def test_explicit_choices_override_the_rules(fb):
    p = plan(fb, workload_desc(fb, 5, 2, waves_per_block=4, chunks_per_block=8))
    assert (p["rows_per_block"], p["chunks_per_block"], p["splits"]) == (256, 8, 17)


def test_range_length_counts_batch_rows(fb):
    # up 4096 -> 11008: 2 chunks at one batch row, 4 at two and four (a group of nb rows
    # counts nb times); the LDS caps four-row ranges at 4 chunks
    assert plan(fb, workload_desc(fb, 4, 0))["chunks_per_block"] == 2
    assert plan(fb, workload_desc(fb, 4, 0, max_batch=2))["chunks_per_block"] == 4
    p = plan(fb, workload_desc(fb, 4, 0, max_batch=4))
    assert p["chunks_per_block"] == 4 and p["splits"] == 17
    # q_proj stays at 2 chunks for two batch rows
    assert plan(fb, workload_desc(fb, 2, 0, max_batch=2))["chunks_per_block"] == 2


def test_matrix_core_plan(fb):
    mf = fb.COMPUTE_MFMA
    # one instance: 256 weight rows per workgroup (grid counted per 32 batch rows)
    p = plan(fb, workload_desc(fb, 4, 0, max_batch=128, compute=mf))
    assert (p["rows_per_block"], p["row_blocks"], p["chunks_per_block"], p["splits"]) == (256, 43, 16, 5)
    assert p["grid"] == 43 * 5
    # 8-chunk ranges up to 64 batch rows, 16 above
    assert plan(fb, workload_desc(fb, 4, 0, max_batch=64, compute=mf))["chunks_per_block"] == 8
    assert plan(fb, workload_desc(fb, 4, 0, max_batch=65, compute=mf))["chunks_per_block"] == 16
    # LDS: two buffers of x (32 batch rows x 136 halfs), c (128 halfs) and 256 rows of sign words
    assert p["lds_bytes"] == 2 * (32 * 136 * 2 + 128 * 2 + 256 * 16)


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
    # the host-side query and a created handle agree (one and four batch rows, matrix cores)
    for lay, kw in [(I.workload_layer(2, 0, 0), {}), (I.workload_layer(4, 1, 0), {"max_batch": 4}),
                    (I.workload_layer(4, 0, 0), {"max_batch": 64, "compute": fb.COMPUTE_MFMA})]:
        dl = fb.DeviceLayer(lay, kw.get("max_batch", 1), compute=kw.get("compute", fb.COMPUTE_LUT))
        d = desc_for(fb, lay.n, lay.k, lay.kb, lay.ks, lay.s, g=lay.g, **kw)
        assert fb.fluxbin_plan_of(d) == dl.plan, (lay.n, lay.k, kw)
        dl.close()
