"""The C-ABI library loads, exports what include/fluxbin.h declares, and validates on the host.

No test here launches a kernel or needs a GPU: every call below is rejected
by host-side validation before any HIP runtime call, or is pure host
arithmetic.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fluxbin.h")


@pytest.fixture(scope="module")
def fb():
    from binary_basis_lut_amd import build as B
    if B.is_stale():
        B.build()
    from binary_basis_lut_amd import fluxbin
    return fluxbin


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fluxbin_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(fb):
    names = declared_functions()
    assert len(names) >= 15
    lib = ctypes.CDLL(str(fb.LIB_PATH))
    for name in names:
        assert hasattr(lib, name), name
    assert sorted(fb.SYMBOLS) == names


def test_abi_version_and_strings(fb):
    assert fb.fluxbin_abi_version() == fb.ABI_VERSION == 8
    assert fb.fluxbin_status_string(fb.OK) == "ok"
    assert "invalid" in fb.fluxbin_status_string(fb.ERR_INVALID_ARGUMENT)
    assert fb.fluxbin_status_string(99) == "unknown status"


@pytest.mark.parametrize("rows,cols", [(1, 1), (64, 128), (65, 129), (4096, 4096), (57344, 8192), (0, 5)])
def test_tiled_words(fb, rows, cols):
    expect = 0 if rows == 0 else -(-rows // 64) * -(-cols // 128) * 256
    assert fb.fluxbin_tiled_words(rows, cols) == expect


def good_desc(fb, **kw):
    d = fb.LayerDesc()
    d.abi_version = fb.ABI_VERSION
    d.g, d.kb, d.ks = 4, 2, 1
    d.n, d.k, d.s, d.max_batch = 4096, 4096, 256, 1
    d.layout = fb.LAYOUT_TILED
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def ws_status(fb, d):
    out = ctypes.c_size_t(0)
    return fb.raw_status("fluxbin_workspace_size", ctypes.byref(d), ctypes.byref(out)), out.value


def test_workspace_size_matches_plan_arithmetic(fb):
    st, ws = ws_status(fb, good_desc(fb))
    assert st == fb.OK
    # 66 chunks of 128 columns (2 x 32 global + 2 salient) over 16 row blocks: split, so one
    # packed 64-bit reduction word per (batch row, padded output row)
    assert ws == 1 * 4096 * 8
    st, ws = ws_status(fb, good_desc(fb, max_batch=4, n=100))
    assert st == fb.OK and ws == 4 * 128 * 8
    # a single 128-column chunk needs no split and no workspace
    st, ws = ws_status(fb, good_desc(fb, k=128, ks=0, s=0, kb=1))
    assert st == fb.OK and ws == 0


def test_too_many_splits_is_unsupported(fb):
    # 255 splits at most: 2 x ceil(2^17 / 128) chunks with one chunk per workgroup is too many
    st, _ = ws_status(fb, good_desc(fb, k=1 << 17, ks=0, s=0, chunks_per_block=1))
    assert st == fb.ERR_UNSUPPORTED


@pytest.mark.parametrize("field,value,status", [
    ("abi_version", 2, 1), ("g", 3, 2), ("g", 16, 2), ("kb", 0, 2), ("kb", 5, 2), ("ks", 3, 2), ("ks", -1, 2),
    ("n", 0, 1), ("k", 0, 1), ("s", 0, 1), ("s", 5000, 1), ("max_batch", 0, 2), ("max_batch", 129, 2),
    ("chunks_per_block", 33, 1), ("chunks_per_block", -1, 1), ("waves_per_block", 2, 1), ("waves_per_block", 16, 1),
    ("row_group", 64, 2), ("row_group", -1, 2), ("sal_group", 8, 1), ("table_precision", 2, 1),
    ("table_precision", -1, 1), ("layout", 2, 1), ("layout", -1, 1),
])
def test_workspace_size_rejects(fb, field, value, status):
    st, _ = ws_status(fb, good_desc(fb, **{field: value}))
    assert st == status, fb.fluxbin_last_error()
    assert fb.fluxbin_last_error()


def test_g8_batch_limit_and_salient_flags(fb):
    assert ws_status(fb, good_desc(fb, g=8, max_batch=4))[0] == fb.OK
    assert ws_status(fb, good_desc(fb, g=8, max_batch=128))[0] == fb.OK  # 32 groups of 4 rows
    assert ws_status(fb, good_desc(fb, g=8, max_batch=129))[0] == fb.ERR_UNSUPPORTED
    # a prefill batch keeps one reduction word per (batch row, padded output row)
    st, ws = ws_status(fb, good_desc(fb, max_batch=128))
    assert st == fb.OK and ws == 128 * 4096 * 8
    assert ws_status(fb, good_desc(fb, ks=0, s=0))[0] == fb.OK
    assert ws_status(fb, good_desc(fb, ks=0, s=8))[0] == fb.ERR_INVALID_ARGUMENT
    # several batch rows: ranges longer than the LDS holds build their tables in groups of chunks
    # (8 rows at g = 4: 20.5 KiB per chunk, groups of 2) ...
    assert ws_status(fb, good_desc(fb, chunks_per_block=8, max_batch=8))[0] == fb.OK
    p = plan_of(fb, good_desc(fb, chunks_per_block=8, max_batch=8))
    assert (p["chunks_per_block"], p["table_chunks"]) == (8, 2) and p["lds_bytes"] == 2 * (8 * 32 * 16 * 4 + 8 * 128 * 4) + 256
    # 16 rows run as two groups of 8 at g = 4 ...
    p = plan_of(fb, good_desc(fb, chunks_per_block=8, max_batch=16))
    assert (p["chunks_per_block"], p["table_chunks"]) == (8, 2)
    # ... but a g = 8 group of 4 rows: the LDS holds one chunk's tables, too few to group
    assert ws_status(fb, good_desc(fb, g=8, chunks_per_block=2, max_batch=4))[0] == fb.ERR_UNSUPPORTED
    # one batch row: the range's tables must fit
    assert ws_status(fb, good_desc(fb, chunks_per_block=32, waves_per_block=8))[0] == fb.ERR_UNSUPPORTED


def plan_of(fb, d):
    info = fb.PlanInfo()
    assert fb.raw_status("fluxbin_plan_of", ctypes.byref(d), ctypes.byref(info)) == fb.OK, fb.fluxbin_last_error()
    return info.as_dict()


def test_column_ranges_never_span_segments(fb):
    # 4096 x 4096, kb = 2, ks = 1, s = 256: 32 global chunks per basis, 2 salient chunks; every
    # segment is cut into ceil(chunks / cpb) ranges, and the longest range is reported
    for cpb, splits, longest in [(1, 66, 1), (2, 33, 2), (3, 2 * 11 + 1, 3), (4, 17, 4), (5, 2 * 7 + 1, 5),
                                 (7, 2 * 5 + 1, 7), (8, 9, 8), (16, 5, 16)]:
        p = plan_of(fb, good_desc(fb, chunks_per_block=cpb, waves_per_block=8))
        assert (p["splits"], p["chunks_per_block"]) == (splits, longest), (cpb, p)
    # 86 chunks (k = 11008) at a target of 7: 13 ranges of 6 or 7 chunks (balanced, never 7 x 12 + 2)
    p = plan_of(fb, good_desc(fb, k=11008, kb=1, ks=0, s=0, chunks_per_block=7, waves_per_block=8))
    assert (p["splits"], p["chunks_per_block"]) == (13, 7)
    # one segment in one range: no split, no workspace
    st, ws = ws_status(fb, good_desc(fb, k=2048, kb=1, ks=0, s=0, chunks_per_block=16, waves_per_block=8))
    assert st == fb.OK and ws == 0
    # the longest range: its tables and inputs within 80 KiB of LDS (31 chunks of 2.5 KiB at g = 4)
    assert ws_status(fb, good_desc(fb, chunks_per_block=31, waves_per_block=4))[0] == fb.OK
    assert ws_status(fb, good_desc(fb, chunks_per_block=32, waves_per_block=8))[0] == fb.ERR_UNSUPPORTED


def test_row_major_inputs_add_their_tiled_copies_to_the_workspace(fb):
    rnd = lambda b: -(-b // 256) * 256
    tiled = ws_status(fb, good_desc(fb))[1]
    st, ws = ws_status(fb, good_desc(fb, layout=fb.LAYOUT_ROWMAJOR))
    assert st == fb.OK
    assert ws == tiled + rnd(2 * fb.fluxbin_tiled_words(4096, 4096) * 4) + rnd(fb.fluxbin_tiled_words(4096, 256) * 4)
    # block-wise scales are converted too: kb blocks with 1 group per chunk, ks with 16 (8 salient per group)
    d = grouped_desc(fb, layout=fb.LAYOUT_ROWMAJOR)
    st, ws = ws_status(fb, d)
    assert st == fb.OK
    expect = (rnd(4096 * 8) + rnd(2 * fb.fluxbin_tiled_words(4096, 4096) * 4) + rnd(2 * fb.fluxbin_tiled_words(4096, 256) * 4)
              + rnd(2 * fb.fluxbin_tiled_scale_elems(4096, 32, 1) * 2) + rnd(2 * fb.fluxbin_tiled_scale_elems(4096, 32, 16) * 2))
    assert ws == expect


def test_create_rejects_before_touching_the_device(fb):
    h = ctypes.c_void_p()
    d = good_desc(fb)  # all pointers NULL
    assert fb.raw_status("fluxbin_create", ctypes.byref(d), ctypes.byref(h)) == fb.ERR_INVALID_ARGUMENT
    assert "non-NULL" in fb.fluxbin_last_error()
    d.bits_global = d.r_global = d.c_global = 0x1000
    d.bits_sal = d.r_sal = d.c_sal = d.sal_idx = 0x2000
    d.bits_global = 0x1004  # misaligned
    assert fb.raw_status("fluxbin_create", ctypes.byref(d), ctypes.byref(h)) == fb.ERR_INVALID_ARGUMENT
    assert "aligned" in fb.fluxbin_last_error()
    d.bits_global = 0x1000
    d.workspace = None
    d.workspace_bytes = 1  # a NULL workspace is accepted only as "none" (0 bytes)
    assert fb.raw_status("fluxbin_create", ctypes.byref(d), ctypes.byref(h)) == fb.ERR_WORKSPACE
    assert fb.raw_status("fluxbin_create", None, ctypes.byref(h)) == fb.ERR_INVALID_ARGUMENT
    assert not h.value


def test_row_major_create_needs_word_alignment_only(fb):
    h = ctypes.c_void_p()
    d = good_desc(fb, layout=fb.LAYOUT_ROWMAJOR)
    d.bits_global = d.r_global = d.c_global = 0x1002
    d.bits_sal = d.r_sal = d.c_sal = d.sal_idx = 0x2000
    assert fb.raw_status("fluxbin_create", ctypes.byref(d), ctypes.byref(h)) == fb.ERR_INVALID_ARGUMENT
    assert "4-byte" in fb.fluxbin_last_error()
    d.bits_global = 0x1004  # 4-byte aligned is enough for row-major words; the workspace check comes next
    d.workspace = None
    assert fb.raw_status("fluxbin_create", ctypes.byref(d), ctypes.byref(h)) == fb.ERR_WORKSPACE
    assert not h.value


def test_reset_and_probes_reject_on_the_host(fb):
    s = fb.raw_status
    assert s("fluxbin_reset_workspace", None, None) == fb.ERR_INVALID_ARGUMENT
    assert s("fluxbin_gemv_static", None, 0x1000, 0x2000, 1, None) == fb.ERR_INVALID_ARGUMENT
    assert s("fluxbin_gemv_timed", None, 0x1000, 0x2000, 1, None, 0x10, 0x20) == fb.ERR_INVALID_ARGUMENT
    assert s("fluxbin_gemv_timed", 0x1000, 0x1000, 0x2000, 1, None, None, 0x20) == fb.ERR_INVALID_ARGUMENT
    I64, I32 = ctypes.c_int64, ctypes.c_int32
    P = 0x1000
    assert s("fluxbin_probe_stream_read", None, I64(1 << 20), I32(4), I64(64), ctypes.c_uint32(0), P, None) == 1
    assert s("fluxbin_probe_stream_read", P, I64(1000), I32(4), I64(64), ctypes.c_uint32(0), P, None) == 1
    assert s("fluxbin_probe_stream_read", P + 8, I64(1 << 20), I32(4), I64(64), ctypes.c_uint32(0), P, None) == 1
    assert s("fluxbin_probe_stream_read", P, I64(1 << 20), I32(3), I64(64), ctypes.c_uint32(0), P, None) == 1
    assert s("fluxbin_probe_stream_read", P, I64(1 << 20), I32(4), I64(0), ctypes.c_uint32(0), P, None) == 1
    assert s("fluxbin_probe_empty", I64(0), I32(64), None) == 1
    assert s("fluxbin_probe_empty", I64(8), I32(2048), None) == 1
    assert s("fluxbin_probe_lds_lookup", I32(4), I32(3), I64(8), I32(1), ctypes.c_float(0), P, None) == 2
    assert s("fluxbin_probe_lds_lookup", I32(8), I32(8), I64(8), I32(1), ctypes.c_float(0), P, None) == 2
    assert s("fluxbin_probe_lds_lookup", I32(4), I32(1), I64(8), I32(0), ctypes.c_float(0), P, None) == 1
    assert s("fluxbin_probe_lds_lookup", I32(4), I32(1), I64(8), I32(1), ctypes.c_float(0), None, None) == 1
    assert s("fluxbin_probe_lds_lookup_banked", I32(3), I64(8), I32(1), ctypes.c_float(0), P, None) == 2
    assert s("fluxbin_probe_lds_lookup_banked", I32(4), I64(0), I32(1), ctypes.c_float(0), P, None) == 1
    assert s("fluxbin_probe_lds_lookup_banked", I32(2), I64(8), I32(1), ctypes.c_float(0), None, None) == 1


def test_launching_calls_reject_bad_arguments_on_the_host(fb):
    s = fb.raw_status
    assert s("fluxbin_gemv", None, 0x1000, 0x2000, 1, None) == fb.ERR_INVALID_ARGUMENT
    assert s("fluxbin_build_lut", None, 0x1000, 1, 0x2000, None) == fb.ERR_INVALID_ARGUMENT
    assert s("fluxbin_destroy", None) == fb.ERR_INVALID_ARGUMENT
    assert s("fluxbin_get_plan", None, None) == fb.ERR_INVALID_ARGUMENT
    assert s("fluxbin_pack", 0x1000, -1, 5, 5, 0, 0x2000, None, None) == fb.ERR_INVALID_ARGUMENT
    assert s("fluxbin_pack", 0x1000, 5, 5, 5, 7, 0x2000, None, None) == fb.ERR_INVALID_ARGUMENT
    assert s("fluxbin_pack", 0x1000, 5, 10, 5, 0, 0x2000, None, None) == fb.ERR_INVALID_ARGUMENT  # ld < cols
    assert s("fluxbin_pack", None, 5, 5, 5, 0, 0x2000, None, None) == fb.ERR_INVALID_ARGUMENT
    assert s("fluxbin_relayout", 0x1000, 5, 5, 0, 3, 0x2000, None) == fb.ERR_INVALID_ARGUMENT
    assert s("fluxbin_relayout", 0x1000, 5, 5, 0, 1, 0x1000, None) == fb.ERR_INVALID_ARGUMENT  # overlap
    assert s("fluxbin_vcm_gather", 0x1000, 4, 0x2000, 5, 5, 9, 0x3000, None) == fb.ERR_INVALID_ARGUMENT
    assert s("fluxbin_vcm_gather", None, 4, 0x2000, 5, 5, 1, 0x3000, None) == fb.ERR_INVALID_ARGUMENT
    assert s("fluxbin_dense_gemv_f16", 0x1000, 8, 12, 0x2000, 0x3000, 1, None) == fb.ERR_UNSUPPORTED
    assert s("fluxbin_dense_gemv_f16", 0x1000, 8, 16, 0x2000, 0x3000, 17, None) == fb.ERR_UNSUPPORTED
    assert s("fluxbin_dense_gemv_f16", 0x1001, 8, 16, 0x2000, 0x3000, 1, None) == fb.ERR_INVALID_ARGUMENT


def test_empty_work_is_a_no_op(fb):
    s = fb.raw_status
    assert s("fluxbin_pack", None, 0, 5, 5, 0, None, None, None) == fb.OK
    assert s("fluxbin_relayout", None, 5, 0, 0, 1, None, None) == fb.OK
    assert s("fluxbin_vcm_gather", None, 0, None, 5, 5, 1, None, None) == fb.OK


@pytest.mark.parametrize("rows,groups,m", [(1, 1, 1), (4096, 32, 1), (4096, 32, 16), (100, 86, 8), (65, 3, 16)])
def test_tiled_scale_elems(fb, rows, groups, m):
    assert fb.fluxbin_tiled_scale_elems(rows, groups, m) == -(-rows // 64) * -(-groups // m) * 64 * m
    assert fb.fluxbin_tiled_scale_elems(rows, groups, 0) == 0
    assert fb.fluxbin_tiled_scale_elems(rows, groups, 129) == 0
    assert fb.fluxbin_tiled_scale_elems(0, groups, m) == 0


def grouped_desc(fb, **kw):
    """q_proj shape in the pages' 2b-s8-g128 storage: 2 + 2 bases, 8 salient columns per 128."""
    base = dict(kb=2, ks=2, s=8 * 32, row_group=128, sal_group=8)
    base.update(kw)
    return good_desc(fb, **base)


def test_block_wise_plan_keeps_global_and_salient_ranges_apart(fb):
    # 2 x 32 global + 2 x 2 salient chunks; with 8 chunks per workgroup: 2 x 4 global ranges + 2 salient ranges
    st, ws = ws_status(fb, grouped_desc(fb, chunks_per_block=8))
    assert st == fb.OK and ws == 4096 * 8
    assert plan_of(fb, grouped_desc(fb, chunks_per_block=8))["splits"] == 10
    # one global chunk (k = 128) and one salient chunk: two ranges, hence a split reduction
    st, ws = ws_status(fb, grouped_desc(fb, k=128, s=8, chunks_per_block=2, kb=1, ks=1))
    assert st == fb.OK and ws == 4096 * 8
    # the same layer without salient bases fits one range and needs no workspace
    st, ws = ws_status(fb, grouped_desc(fb, k=128, s=0, ks=0, sal_group=0, chunks_per_block=2, kb=1))
    assert st == fb.OK and ws == 0


@pytest.mark.parametrize("kw,status", [
    (dict(sal_group=4), 2), (dict(sal_group=32), 2), (dict(sal_group=0), 2), (dict(s=255), 1), (dict(s=512), 1),
    (dict(g=8, sal_group=8), 0), (dict(g=8, sal_group=16, s=16 * 32), 0), (dict(ks=0, s=0, sal_group=0), 0),
    (dict(ks=0, s=0, sal_group=8), 1), (dict(k=300, s=8 * 3), 0), (dict(k=300, s=8 * 2), 1),
])
def test_block_wise_desc_validation(fb, kw, status):
    st, _ = ws_status(fb, grouped_desc(fb, **kw))
    assert st == status, fb.fluxbin_last_error()


def test_relayout_scales_rejects_on_the_host(fb):
    s = fb.raw_status
    assert s("fluxbin_relayout_scales", 0x1000, 5, 5, 0, 0, 1, 0x2000, None) == fb.ERR_INVALID_ARGUMENT  # m = 0
    assert s("fluxbin_relayout_scales", 0x1000, 5, 5, 129, 0, 1, 0x2000, None) == fb.ERR_INVALID_ARGUMENT
    assert s("fluxbin_relayout_scales", 0x1000, 5, 5, 1, 0, 2, 0x2000, None) == fb.ERR_INVALID_ARGUMENT
    assert s("fluxbin_relayout_scales", 0x1000, 5, 5, 1, 0, 1, 0x1000, None) == fb.ERR_INVALID_ARGUMENT
    assert s("fluxbin_relayout_scales", None, 5, 5, 1, 0, 1, 0x2000, None) == fb.ERR_INVALID_ARGUMENT
    assert s("fluxbin_relayout_scales", None, 0, 5, 1, 0, 1, None, None) == fb.OK


def test_block_wise_create_checks_salient_scale_alignment(fb):
    h = ctypes.c_void_p()
    d = grouped_desc(fb)
    d.bits_global = d.r_global = d.c_global = 0x1000
    d.bits_sal = d.c_sal = d.sal_idx = 0x2000
    d.r_sal = 0x2002
    assert fb.raw_status("fluxbin_create", ctypes.byref(d), ctypes.byref(h)) == fb.ERR_INVALID_ARGUMENT
    assert "r_sal" in fb.fluxbin_last_error()


def test_decomposition_host_validation(fb):
    s = fb.raw_status
    out = ctypes.c_size_t(0)
    assert s("fluxbin_decomp_workspace_size", 4096, 4096, 2, ctypes.byref(out)) == fb.OK
    assert out.value == 8 * (64 * 4096 + 1024 + 16 + 4 * 8192)
    assert s("fluxbin_decomp_workspace_size", 4096, 4096, 5, ctypes.byref(out)) == fb.ERR_UNSUPPORTED
    assert s("fluxbin_decomp_workspace_size", 0, 4096, 2, ctypes.byref(out)) == fb.ERR_INVALID_ARGUMENT
    assert s("fluxbin_decomp_workspace_size", (1 << 22) + 1, 8, 2, ctypes.byref(out)) == fb.ERR_UNSUPPORTED
    assert s("fluxbin_decomp_workspace_size", 8, 8, 2, None) == fb.ERR_INVALID_ARGUMENT
    P = 0x1000
    # basis out of range, NULL pointers, missing workspace
    assert s("fluxbin_decomp_row_scales", P, 8, 8, 2, 2, P, P, P, None, P, P, 1 << 20, None) == fb.ERR_INVALID_ARGUMENT
    assert s("fluxbin_decomp_row_scales", None, 8, 8, 2, 0, P, P, P, None, P, P, 1 << 20, None) == fb.ERR_INVALID_ARGUMENT
    assert s("fluxbin_decomp_row_scales", P, 8, 8, 2, 0, P, P, P, None, P, None, 0, None) == fb.ERR_WORKSPACE
    assert s("fluxbin_decomp_row_scales", P, 8, 8, 2, 0, P, P, P, None, P, P, 16, None) == fb.ERR_WORKSPACE
    assert s("fluxbin_decomp_row_scales", P, 8, 8, 2, 0, P, P, P, None, P, P + 8, 1 << 20, None) == \
        fb.ERR_INVALID_ARGUMENT  # misaligned workspace
    assert s("fluxbin_decomp_col_scales", P, 8, 8, 2, -1, P, P, P, P, P, 1 << 20, None) == fb.ERR_INVALID_ARGUMENT
    assert s("fluxbin_decomp_signs", P, 8, 8, 0, P, P, P, None) == fb.ERR_UNSUPPORTED
    assert s("fluxbin_decomp_signs", P, 8, 8, 2, None, P, P, None) == fb.ERR_INVALID_ARGUMENT
    assert s("fluxbin_decomp_residual_signs", P, 8, 8, 2, 3, P, P, P, P, None) == fb.ERR_INVALID_ARGUMENT
    assert s("fluxbin_decomp_error", P, 8, 8, 2, P, P, P, None, None, P, 1 << 20, None) == fb.ERR_INVALID_ARGUMENT
    assert s("fluxbin_decompose", P, 8, 8, 2, -1, None, P, P, P, P, P, None, P, 1 << 20, None) == \
        fb.ERR_INVALID_ARGUMENT
    assert s("fluxbin_decompose", P, 8, 8, 2, 3, None, P, P, None, P, P, None, P, 1 << 20, None) == \
        fb.ERR_INVALID_ARGUMENT
    assert s("fluxbin_decompose", P, 8, 8, 2, 3, None, P, P, P, P, P, None, P, 100, None) == fb.ERR_WORKSPACE
