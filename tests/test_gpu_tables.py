"""GPU parity of the fp16-table GEMV (quantised tables, LUT Tensor Core notes, section 3.1.3).

The contract of this format (what the tests hold the kernel to):
  * against the exact product (the oracle's fp64 dense route): |y - y_exact| <= (2^-11 + g 2^-24) M
    plus the rigorous fp32 accumulation + fp16 output bound of test_gpu_parity, with
    M = sum over segments of |r| * sum |c x|.  This is the format's own tolerance, looser than the
    1e-3 * sum|W_hat x| contract of the fp32 tables: each entry is one fp16 rounding of a sum of g
    terms;
  * dyadic inputs (every entry exact in fp16): y equal to RNE(exact), bitwise.

A diagnostic, not the contract: the oracle's LUT route with fp16 entries built the way the kernel
builds them (fp32 sum in the kernel's order, rounded to fp16 once) quantises every entry like the
kernel, so the kernel must also sit within the plain accumulation bound of that route.  That
route mirrors the kernel's entry arithmetic, so it pins nothing by itself; it only localises a
failure (table build versus accumulation) when the contract check fails.
"""
import numpy as np
import pytest

from binary_basis_lut_amd import inputs as I

from .test_gpu_parity import gemv, magnitude, note

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def fb():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    from binary_basis_lut_amd import fluxbin
    return fluxbin


def check_fp16_tables(orc, layer, x, y16, plan, rows=None):
    rows = np.arange(layer.n) if rows is None else np.asarray(rows)
    y = orc.half_to_double(y16[:, rows])
    assert np.all(np.isfinite(y))
    y_ex, mag = orc.gemv_dense(layer, x, rows=rows)
    M = magnitude(layer, x, rows)
    steps = layer.g + max(layer.k, layer.s) / layer.g + layer.kb + layer.ks + plan["splits"] + 3
    fp32 = 2.0 ** -24 * steps * M + plan["splits"] * 2.0 ** -30
    # the contract: the exact product within the format's quantisation tolerance
    tight_ex = 2.0 ** -11 * (np.abs(y_ex) + fp32) * (1 + 2.0 ** -23) + fp32 + 2.0 ** -25
    quant = (2.0 ** -11 + layer.g * 2.0 ** -24) * M + tight_ex
    err = np.abs(y - y_ex)
    assert np.all(err <= quant), f"contract (vs exact product): worst ratio {float((err / quant).max()):.3g}"
    # diagnostic: the kernel-order fp16 tables of the oracle's LUT route, accumulation bound only
    y_q = orc.gemv_lut_fp16_tables(layer, x, rows=rows)
    tight = 2.0 ** -11 * (np.abs(y_q) + fp32) * (1 + 2.0 ** -23) + fp32 + 2.0 ** -25
    err_q = np.abs(y - y_q)
    assert np.all(err_q <= tight), f"diagnostic (vs kernel-order fp16 tables): worst ratio {float((err_q / tight).max()):.3g}"
    return float((err / quant).max()), float((err_q / tight).max())


EXACT = [
    # g, n, k, kb, ks, s, batch, blockwise sal_group (0: per-row)
    (4, 300, 1000, 2, 1, 77, 1, 0),
    (4, 130, 4096, 2, 1, 256, 16, 0),
    # batch-row pairs of fp16 tables: one pair (2 rows), and 3 rows in a 4-row workgroup (the
    # second pair's high half belongs to no row)
    (4, 200, 1000, 2, 1, 77, 2, 0),
    (4, 150, 777, 2, 1, 40, 3, 0),
    (8, 200, 4096, 3, 1, 96, 1, 0),
    (8, 64, 257, 1, 2, 31, 4, 0),
    (4, 130, 4096, 2, 2, 0, 3, 8),
    (8, 64, 384, 1, 2, 0, 2, 16),
]


@pytest.mark.parametrize("g,n,k,kb,ks,s,batch,sg", EXACT)
def test_fp16_tables_exact_dyadic(fb, orc, g, n, k, kb, ks, s, batch, sg):
    note(f"fp16 tables exact g={g} n={n} k={k} kb={kb} ks={ks} batch={batch} sal_group={sg}")
    if sg:
        layer = I.dyadic_grouped_layer(n, k, kb, ks, g, 128, sg, seed=n + k)
    else:
        layer = I.dyadic_layer(n, k, kb, ks, g, s, seed=n + k)
    x = I.dyadic_x(k, batch, seed=k + batch)
    dl = fb.DeviceLayer(layer, max_batch=batch, table_precision=fb.TABLE_F16)
    y16 = gemv(fb, dl, x)
    y_ref, _ = orc.gemv_dense(layer, x)
    assert np.array_equal(y16, orc.double_to_half(y_ref))
    dl.close()


SHAPES = [
    # name, cid, shape_idx, batch, blockwise sal_group
    ("q_proj", 2, 0, 1, 0),
    ("q_proj_b16", 2, 0, 16, 0),
    ("7b_qkv_g8", 3, 0, 1, 0),
    ("7b_down_g8_b4", 3, 3, 4, 0),
    ("70b_gate_up", 5, 2, 1, 0),
    ("70b_down", 5, 3, 1, 0),
    ("q_proj_blockwise_s8", 2, 0, 1, 8),
]


@pytest.mark.parametrize("name,cid,shape_idx,batch,sg", SHAPES)
def test_fp16_tables_workloads(fb, orc, name, cid, shape_idx, batch, sg):
    note(f"fp16 tables {name}")
    if sg:
        sh = I.WORKLOADS[cid].shapes[shape_idx]
        layer = I.make_grouped_layer(sh.n, sh.k, 2, 2, I.WORKLOADS[cid].g, 128, sg, outlier_frac=0.01,
                                     seed=(cid, 0, 100 + sg))
        x = I.make_x(layer, batch, seed=(cid, 0, 100 + sg))
    else:
        layer = I.workload_layer(cid, shape_idx)
        x = I.workload_x(cid, layer, batch, shape_idx)
    dl = fb.DeviceLayer(layer, max_batch=batch, table_precision=fb.TABLE_F16)
    y16 = gemv(fb, dl, x)
    n = layer.n
    rows = None if n <= 4096 else np.unique(np.concatenate([np.arange(32), np.arange(n - 32, n),
                                                             I.stream(110, n).choice(n, 256, replace=False)]))
    r = check_fp16_tables(orc, layer, x, y16, dl.plan, rows)
    print(name, "plan", dl.plan, "ratios (contract vs exact / diagnostic vs kernel-order tables):", r)
    dl.close()


@pytest.mark.parametrize("g,n,k,kb,ks,s,batch,cpb,waves", [(4, 4096, 4096, 2, 1, 256, 1, 1, 0),
                                                           (4, 4096, 4096, 2, 1, 256, 1, 32, 8),
                                                           (4, 777, 1031, 4, 2, 500, 16, 0, 0),
                                                           (8, 4096, 4096, 3, 1, 96, 2, 4, 8),
                                                           (8, 100, 1000, 4, 2, 999, 3, 0, 0)])
def test_fp16_tables_edge_cases(fb, orc, g, n, k, kb, ks, s, batch, cpb, waves):
    note(f"fp16 tables edge g={g} n={n} k={k} batch={batch} cpb={cpb} waves={waves}")
    layer = I.make_layer(n, k, kb, ks, g, s=s, outlier_frac=0.01, seed=(111, n, k))
    x = I.make_x(layer, batch, seed=(111, n, k))
    dl = fb.DeviceLayer(layer, max_batch=batch, chunks_per_block=cpb, waves_per_block=waves,
                        table_precision=fb.TABLE_F16)
    y16 = gemv(fb, dl, x)
    check_fp16_tables(orc, layer, x, y16, dl.plan)
    dl.close()


def test_fp16_tables_halve_the_lds_per_chunk(fb):
    layer = I.workload_layer(2)
    a = fb.DeviceLayer(layer, max_batch=8, chunks_per_block=2)
    b = fb.DeviceLayer(layer, max_batch=8, chunks_per_block=2, table_precision=fb.TABLE_F16)
    sink = 256
    # per chunk: 8 batch rows x 32 tables x 16 entries (4 or 2 bytes) + 8 x 128 fp32 inputs
    assert a.plan["lds_bytes"] - sink == 2 * (8 * 32 * 16 * 4 + 8 * 128 * 4)
    assert b.plan["lds_bytes"] - sink == 2 * (8 * 32 * 16 * 2 + 8 * 128 * 4)
    a.close()
    b.close()
