"""GPU parity at prefill-size batches (32..128 rows): batches wider than one workgroup's table set
(8 rows at g = 4, 4 at g = 8) run as batch groups.  Bars as in test_gpu_parity: the contract and
the rounding bound on sampled rows, RNE(exact) on dyadic inputs, and every batch row bitwise equal
to the batch-1 result of the same handle.
"""
import numpy as np
import pytest

from binary_basis_lut_amd import inputs as I

from .test_gpu_parity import check_y, gemv, note

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def fb():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    from binary_basis_lut_amd import fluxbin
    return fluxbin


CASES = [
    # name, k, n, g, kb, ks, s, batch, blockwise
    ("mlp_up_b128", 4096, 11008, 4, 2, 1, 96, 128, False),
    ("mlp_down_b64", 11008, 4096, 4, 2, 1, 224, 64, False),
    ("q_proj_b33", 4096, 4096, 4, 2, 1, 256, 33, False),
    ("g8_b37", 4096, 4096, 8, 3, 1, 96, 37, False),
    ("q_proj_blockwise_b100", 4096, 4096, 4, 2, 2, 8, 100, True),
]


@pytest.mark.parametrize("name,k,n,g,kb,ks,s,batch,blockwise", CASES)
def test_prefill_batches(fb, orc, name, k, n, g, kb, ks, s, batch, blockwise):
    note(f"prefill {name}: k={k} n={n} g={g} kb={kb} ks={ks} batch={batch}")
    if blockwise:
        layer = I.make_grouped_layer(n, k, kb, ks, g, 128, s, outlier_frac=0.01, seed=(96, n, k))
    else:
        layer = I.make_layer(n, k, kb, ks, g, s=s, outlier_frac=0.01, seed=(96, n, k))
    x = I.make_x(layer, batch, seed=(96, n, k))
    dl = fb.DeviceLayer(layer, max_batch=batch)
    y16 = gemv(fb, dl, x)
    rows = np.unique(np.concatenate([np.arange(32), np.arange(n - 32, n),
                                     I.stream(97, n, batch).choice(n, 160, replace=False)]))
    r = check_y(orc, layer, x, y16, dl.plan, rows=rows)
    print(name, "plan", dl.plan, "ratios:", r)
    for b in (0, batch // 2, batch - 1):
        assert np.array_equal(gemv(fb, dl, x[b:b + 1])[0], y16[b])
    dl.close()


@pytest.mark.parametrize("g,n,k,kb,ks,s,batch", [(4, 130, 1000, 2, 1, 77, 40), (8, 64, 257, 1, 2, 31, 10),
                                                 (4, 65, 129, 4, 2, 129, 128)])
def test_prefill_exact_dyadic(fb, orc, g, n, k, kb, ks, s, batch):
    note(f"prefill exact g={g} n={n} k={k} batch={batch}")
    layer = I.dyadic_layer(n, k, kb, ks, g, s, seed=n + k + batch)
    x = I.dyadic_x(k, batch, seed=k + batch)
    dl = fb.DeviceLayer(layer, max_batch=batch)
    y16 = gemv(fb, dl, x)
    y_ref, _ = orc.gemv_dense(layer, x)
    assert np.array_equal(y16, orc.double_to_half(y_ref))
    dl.close()


# Several batch rows with column ranges longer than the LDS holds: the tables are built in groups of
# table_chunks chunks in turn (a group of 2 at 8 rows of g = 4, 4 at 4 rows, 12 at 2 rows, 2 at g = 8
# with 2 rows, 4 with 8 rows of fp16 tables; 16 rows run as two groups of 8).  Last groups shorter than a group and than the
# prefetch depth, salient ranges, block-wise scales, both workgroup sizes.  Dyadic inputs must give
# RNE(exact); random inputs the contract and the rounding bound; batch rows equal the batch-1 call.
GROUPED = [
    # g, n, k, kb, ks, s, batch, cpb, waves, blockwise sal_group, fp16 tables
    (4, 700, 4096, 2, 1, 256, 8, 8, 0, 0, False),
    (4, 700, 4096, 2, 1, 256, 5, 5, 8, 0, False),
    (4, 700, 4096, 2, 1, 256, 8, 16, 4, 0, False),
    (4, 300, 11008, 2, 1, 224, 4, 16, 8, 0, False),
    (4, 300, 4096, 3, 2, 1000, 2, 16, 4, 0, False),
    (4, 300, 4096, 2, 1, 256, 16, 8, 0, 0, True),
    (4, 500, 4096, 2, 2, 0, 8, 8, 0, 8, False),
    (4, 500, 4096, 2, 2, 0, 6, 5, 8, 16, False),
    (8, 300, 4096, 3, 1, 96, 2, 4, 8, 0, False),
    (8, 300, 4096, 3, 1, 96, 2, 5, 0, 0, False),
]


@pytest.mark.parametrize("g,n,k,kb,ks,s,batch,cpb,waves,sg,f16", GROUPED)
def test_grouped_tables(fb, orc, g, n, k, kb, ks, s, batch, cpb, waves, sg, f16):
    note(f"grouped tables g={g} n={n} k={k} kb={kb} ks={ks} batch={batch} cpb={cpb} waves={waves} sg={sg} f16={f16}")
    tp = fb.TABLE_F16 if f16 else fb.TABLE_F32
    if sg:
        layer = I.dyadic_grouped_layer(n, k, kb, ks, g, 128, sg, seed=n + k + batch)
    else:
        layer = I.dyadic_layer(n, k, kb, ks, g, s, seed=n + k + batch)
    x = I.dyadic_x(k, batch, seed=k + batch)
    dl = fb.DeviceLayer(layer, max_batch=batch, chunks_per_block=cpb, waves_per_block=waves, table_precision=tp)
    assert dl.plan["table_chunks"] < dl.plan["chunks_per_block"] <= cpb, dl.plan
    y16 = gemv(fb, dl, x)
    y_ref, _ = orc.gemv_dense(layer, x)
    assert np.array_equal(y16, orc.double_to_half(y_ref)), "y differs from RNE(exact)"
    dl.close()
    if sg:
        layer = I.make_grouped_layer(n, k, kb, ks, g, 128, sg, outlier_frac=0.01, seed=(98, n, k))
    else:
        layer = I.make_layer(n, k, kb, ks, g, s=s, outlier_frac=0.01, seed=(98, n, k))
    x = I.make_x(layer, batch, seed=(98, n, k))
    dl = fb.DeviceLayer(layer, max_batch=batch, chunks_per_block=cpb, waves_per_block=waves, table_precision=tp)
    y16 = gemv(fb, dl, x)
    if f16:
        from .test_gpu_tables import check_fp16_tables
        check_fp16_tables(orc, layer, x, y16, dl.plan)
    else:
        check_y(orc, layer, x, y16, dl.plan)
    for b in (0, batch - 1):
        assert np.array_equal(gemv(fb, dl, x[b:b + 1])[0], y16[b])
    dl.close()
