"""GPU parity of the block-wise row-scale format (one fp16 row scale per row per basis per
128-column group, s salient columns per group: the storage of the FluxBin summary, appendix C.2)
through the C ABI, against the fp64 oracle.  Bars as in test_gpu_parity: bit-exact scale relayout,
y bit-identical to RNE(exact) on dyadic inputs, and the per-row contract plus the rounding bound.
"""
import numpy as np
import pytest

from binary_basis_lut_amd import inputs as I

from .test_gpu_parity import check_y, dev, gemv, host_u16, note

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def fb():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    from binary_basis_lut_amd import fluxbin
    return fluxbin


@pytest.mark.parametrize("rows,groups,m", [(1, 1, 1), (64, 32, 1), (65, 33, 1), (4096, 32, 16), (100, 86, 16),
                                           (7, 5, 8), (300, 64, 8)])
def test_relayout_scales_bit_exact(fb, orc, rows, groups, m):
    note(f"relayout_scales rows={rows} groups={groups} m={m}")
    canon = I.stream(70, rows, groups, m).integers(0, 1 << 16, size=(rows, groups)).astype(np.uint16)
    src = dev(canon, np.int16)
    te = fb.fluxbin_tiled_scale_elems(rows, groups, m)
    tiled = torch.full((te,), -1, dtype=torch.int16, device="cuda")
    fb.fluxbin_relayout_scales(src, rows, groups, m, fb.LAYOUT_ROWMAJOR, fb.LAYOUT_TILED, tiled)
    back = torch.full_like(src, -1)
    fb.fluxbin_relayout_scales(tiled, rows, groups, m, fb.LAYOUT_TILED, fb.LAYOUT_ROWMAJOR, back)
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(tiled), orc.tile_scales(canon, m))
    assert np.array_equal(host_u16(back), canon)


EXACT = [
    # g, n, k, kb, ks, sal_group, batch
    (4, 300, 1000, 2, 2, 8, 1),
    (4, 130, 4096, 2, 2, 8, 16),
    (4, 65, 136, 4, 2, 8, 3),
    (4, 64, 512, 2, 1, 16, 2),
    (4, 1, 128, 1, 0, 0, 1),
    (8, 200, 4096, 3, 1, 16, 1),
    (8, 64, 384, 1, 2, 8, 4),
]


@pytest.mark.parametrize("g,n,k,kb,ks,sg,batch", EXACT)
def test_grouped_exact_dyadic(fb, orc, g, n, k, kb, ks, sg, batch):
    note(f"block-wise exact g={g} n={n} k={k} kb={kb} ks={ks} sal_group={sg} batch={batch}")
    layer = I.dyadic_grouped_layer(n, k, kb, ks, g, 128, sg or 8, seed=n + k)
    x = I.dyadic_x(k, batch, seed=k + batch + 1)
    dl = fb.DeviceLayer(layer, max_batch=batch)
    y16 = gemv(fb, dl, x)
    y_ref, _ = orc.gemv_dense(layer, x)
    assert np.array_equal(y16, orc.double_to_half(y_ref)), "y differs from RNE(exact)"
    dl.close()


# The pages' storage formats at the LLaMA-2 shapes (synthetic values): 2 global + 2 salient bases,
# 8 or 16 salient columns per 128 (about 2.63 / 2.75 bits per weight).
SHAPES = [
    # name, k, n, g, kb, ks, sal_group, batch
    ("q_proj_s8", 4096, 4096, 4, 2, 2, 8, 1),
    ("q_proj_s16", 4096, 4096, 4, 2, 2, 16, 1),
    ("q_proj_kb2_only", 4096, 4096, 4, 2, 0, 0, 1),
    ("70b_gate_up_s8", 8192, 57344, 4, 2, 2, 8, 1),
    ("70b_down_s8", 28672, 8192, 4, 2, 2, 8, 1),
    ("7b_mlp_up_s8_b16", 4096, 11008, 4, 2, 2, 8, 16),
    ("7b_qkv_g8_s16", 4096, 12288, 8, 3, 1, 16, 1),
]


@pytest.mark.parametrize("name,k,n,g,kb,ks,sg,batch", SHAPES)
def test_grouped_shapes(fb, orc, name, k, n, g, kb, ks, sg, batch):
    note(f"block-wise shape {name}: k={k} n={n} g={g} kb={kb} ks={ks} sal_group={sg} batch={batch}")
    layer = I.make_grouped_layer(n, k, kb, ks, g, 128, sg or 8, outlier_frac=0.01, seed=(71, n, k))
    x = I.make_x(layer, batch, seed=(71, n, k))
    dl = fb.DeviceLayer(layer, max_batch=batch)
    y16 = gemv(fb, dl, x)
    rows = None if n <= 4096 else np.unique(np.concatenate([np.arange(64), np.arange(n - 64, n),
                                                             I.stream(72, n).choice(n, 512, replace=False)]))
    r = check_y(orc, layer, x, y16, dl.plan, rows=rows)
    print(name, "plan", dl.plan, "ratios (contract, tight):", r)
    dl.close()


EDGE = [
    # g, n, k, kb, ks, sal_group, batch, cpb, waves
    (4, 63, 136, 1, 1, 8, 1, 0, 0),
    (4, 4096, 4096, 2, 2, 8, 1, 1, 0),
    (4, 4096, 4096, 2, 2, 8, 1, 2, 0),
    (4, 4096, 4096, 2, 2, 8, 1, 3, 0),
    (4, 4096, 4096, 2, 2, 8, 1, 8, 0),
    (4, 4096, 4096, 2, 2, 16, 1, 16, 4),
    (4, 4096, 4096, 2, 2, 8, 1, 31, 8),
    (4, 777, 1032, 4, 2, 8, 16, 0, 0),
    (4, 2000, 1000, 2, 1, 16, 5, 3, 8),
    (4, 257, 11008, 2, 2, 8, 8, 2, 0),
    (4, 300, 2560, 3, 2, 16, 2, 9, 8),
    (8, 100, 1000, 4, 2, 8, 3, 0, 0),
    (8, 4096, 4096, 3, 1, 8, 1, 1, 0),
    (8, 4096, 4096, 3, 1, 16, 2, 2, 8),
]


@pytest.mark.parametrize("g,n,k,kb,ks,sg,batch,cpb,waves", EDGE)
def test_grouped_edge_cases(fb, orc, g, n, k, kb, ks, sg, batch, cpb, waves):
    note(f"block-wise edge g={g} n={n} k={k} kb={kb} ks={ks} sal_group={sg} batch={batch} cpb={cpb} "
         f"waves={waves}")
    layer = I.make_grouped_layer(n, k, kb, ks, g, 128, sg, outlier_frac=0.01, seed=(73, n, k))
    x = I.make_x(layer, batch, seed=(73, n, k))
    dl = fb.DeviceLayer(layer, max_batch=batch, chunks_per_block=cpb, waves_per_block=waves)
    y16 = gemv(fb, dl, x)
    check_y(orc, layer, x, y16, dl.plan)
    dl.close()


def test_grouped_batch_rows_match_single_calls(fb):
    note("block-wise batch 16 vs batch 1 rows")
    layer = I.make_grouped_layer(4096, 4096, 2, 2, 4, 128, 8, seed=(74, 0, 0))
    dl = fb.DeviceLayer(layer, max_batch=16)
    x16 = I.make_x(layer, 16, seed=(74, 0, 0))
    y16 = gemv(fb, dl, x16)
    for b in (0, 9, 15):
        assert np.array_equal(gemv(fb, dl, x16[b:b + 1])[0], y16[b])
    dl.close()


def test_grouped_create_rejects_unstructured_salient_set(fb):
    layer = I.make_grouped_layer(128, 512, 1, 1, 4, 128, 8, seed=(75, 0, 0))
    idx = layer.sal_idx.copy()
    # the last salient column of group 0 moves to an unused column of group 1: still strictly
    # ascending and in range, but group 0 now has 7 salient columns and group 1 has 9
    idx[7] = np.setdiff1d(np.arange(128, 256), idx)[0]
    idx = np.sort(idx)
    assert np.all(np.diff(idx) > 0) and np.bincount(idx // 128, minlength=4)[0] == 7
    layer.sal_idx = idx.astype(np.int32)
    with pytest.raises(fb.FluxbinError) as ei:
        fb.DeviceLayer(layer)
    assert ei.value.status == fb.ERR_INVALID_ARGUMENT
