"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Bars:
  * packing, relayout and VCM gathers: bit-exact;
  * tables: within (g-1) * 2^-24 * sum_t |v_t| of the exact entry;
  * y: the contract |y - y_ref| <= 1e-3 * sum_j |W_hat_ij x_j| per row, and the
    rigorous first-order fp32/fp16 bound below; with dyadic inputs (every
    partial sum exact in fp32) y must equal RNE-to-fp16 of the exact value.
"""
import os

import numpy as np
import pytest

from binary_basis_lut_amd import inputs as I

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def fb():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    from binary_basis_lut_amd import fluxbin
    return fluxbin


def note(msg):
    print(f"[case] {msg}", flush=True)


def dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a).view(dtype)).cuda()


def host_u16(t):
    return t.cpu().numpy().view(np.uint16)


def gemv(fb, dl, x_np):
    x = dev(x_np, np.int16)
    y = torch.full((x_np.shape[0], dl.layer.n), 0x7e00, dtype=torch.int16, device="cuda")  # NaN sentinel
    dl.gemv(x, y)
    torch.cuda.synchronize()
    return host_u16(y)


def magnitude(layer, x_np, rows):
    """sum over segments of |r| * sum_cols |c * x|: the scale of every fp32 rounding in one row
    (block-wise row scales: the sum over groups of |r| * the group's sum of |c * x|)."""
    xd = x_np.view(np.float16).astype(np.float64)
    out = np.zeros((xd.shape[0], len(rows)))
    if getattr(layer, "row_group", 0):
        G = layer.row_group
        for b in range(layer.kb):
            cx = np.abs(xd) * np.abs(layer.c_g[b].view(np.float16).astype(np.float64))[None, :]
            grp = np.add.reduceat(cx, np.arange(0, layer.k, G), axis=1)                     # [batch][groups]
            out += grp @ np.abs(layer.r_g[b][rows].view(np.float16).astype(np.float64)).T
        for b in range(layer.ks):
            cx = np.abs(xd[:, layer.sal_idx]) * np.abs(layer.c_s[b].view(np.float16).astype(np.float64))[None, :]
            grp = np.zeros((xd.shape[0], -(-layer.k // G)))
            np.add.at(grp.T, layer.sal_idx // G, cx.T)
            out += grp @ np.abs(layer.r_s[b][rows].view(np.float16).astype(np.float64)).T
        return out
    for b in range(layer.kb):
        a = np.abs(xd) @ np.abs(layer.c_g[b].view(np.float16).astype(np.float64))
        out += np.abs(layer.r_g[b][rows].view(np.float16).astype(np.float64))[None, :] * a[:, None]
    for b in range(layer.ks):
        a = np.abs(xd[:, layer.sal_idx]) @ np.abs(layer.c_s[b].view(np.float16).astype(np.float64))
        out += np.abs(layer.r_s[b][rows].view(np.float16).astype(np.float64))[None, :] * a[:, None]
    return out


def check_y(orc, layer, x_np, y16, plan, rows=None, steps=None):
    """Assert the contract and the rigorous bound on the listed rows; return the worst ratios.

    `steps` bounds the fp32 roundings any one product term goes through (default: the LUT route's
    table build, one lookup add per g columns, the scale folds and the split partials)."""
    rows = np.arange(layer.n) if rows is None else np.asarray(rows)
    y_ref, mag = orc.gemv_dense(layer, x_np, rows=rows)
    y = orc.half_to_double(y16[:, rows])
    err = np.abs(y - y_ref)
    assert np.all(np.isfinite(y)), "non-finite output"
    contract = 1e-3 * mag
    if steps is None:
        steps = layer.g + max(layer.k, layer.s) / layer.g + layer.kb + layer.ks + plan["splits"] + 3
    # fp32 table build and accumulation (first-order worst case), fixed-point combination of the
    # split partials (2^-30 per partial, exact sum), then fp16 output rounding (possibly via fp32)
    fp32 = 2.0 ** -24 * steps * magnitude(layer, x_np, rows) + plan["splits"] * 2.0 ** -30
    tight = 2.0 ** -11 * (np.abs(y_ref) + fp32) * (1 + 2.0 ** -23) + fp32 + 2.0 ** -25
    bad = err > contract
    assert not bad.any(), f"contract violated at {np.argwhere(bad)[:5]}: err {err[bad][:5]} tol {contract[bad][:5]}"
    bad = err > tight
    assert not bad.any(), f"rounding bound violated at {np.argwhere(bad)[:5]}: err {err[bad][:5]} tol {tight[bad][:5]}"
    return float((err / np.maximum(contract, 1e-300)).max()), float((err / tight).max())


# ----------------------------------------------------------------------------- bit-exact helpers

@pytest.mark.parametrize("rows,cols", [(1, 1), (3, 31), (64, 128), (65, 129), (200, 1000), (130, 4096)])
def test_pack_bit_exact(fb, orc, rows, cols):
    note(f"pack rows={rows} cols={cols}")
    rng = np.random.default_rng(rows * 7 + cols)
    ld = cols + 3
    signs = rng.choice(np.array([-1, 1], np.int8), size=(rows, ld))
    signs[rows // 2, 0] = 0
    signs[-1, cols - 1] = 9
    signs[0, cols:] = 77  # beyond cols: ignored
    ref, bad = orc.pack_rowmajor(signs[:, :cols])
    n_bad = int(((signs[:, :cols] != 1) & (signs[:, :cols] != -1)).sum())
    assert bad == n_bad
    s_dev = dev(signs, np.int8)
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.full((rows * ((cols + 31) // 32),), -1, dtype=torch.int32, device="cuda")
    fb.fluxbin_pack(s_dev, rows, cols, ld, fb.LAYOUT_ROWMAJOR, out, cnt)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32).reshape(ref.shape), ref)
    assert int(cnt.item()) == n_bad
    tw = fb.fluxbin_tiled_words(rows, cols)
    out_t = torch.full((tw,), -1, dtype=torch.int32, device="cuda")
    fb.fluxbin_pack(s_dev, rows, cols, ld, fb.LAYOUT_TILED, out_t, None)
    torch.cuda.synchronize()
    assert np.array_equal(out_t.cpu().numpy().view(np.uint32), orc.tile_words(ref, cols))


@pytest.mark.parametrize("rows,cols", [(1, 1), (63, 33), (64, 128), (129, 300), (4096, 256)])
def test_relayout_bit_exact(fb, orc, rows, cols):
    note(f"relayout rows={rows} cols={cols}")
    canon = I.sign_words(I.stream(50, rows, cols), rows, cols)
    src = dev(canon, np.int32)
    tw = fb.fluxbin_tiled_words(rows, cols)
    tiled = torch.full((tw,), -1, dtype=torch.int32, device="cuda")
    fb.fluxbin_relayout(src, rows, cols, fb.LAYOUT_ROWMAJOR, fb.LAYOUT_TILED, tiled)
    back = torch.full_like(src, -1)
    fb.fluxbin_relayout(tiled, rows, cols, fb.LAYOUT_TILED, fb.LAYOUT_ROWMAJOR, back)
    torch.cuda.synchronize()
    assert np.array_equal(tiled.cpu().numpy().view(np.uint32), orc.tile_words(canon, cols))
    assert np.array_equal(back.cpu().numpy().view(np.uint32), canon)


@pytest.mark.parametrize("k,s,rows", [(64, 10, 9), (4096, 256, 300), (11008, 224, 40), (100, 100, 3), (33, 1, 5)])
def test_vcm_gather_bit_exact(fb, orc, k, s, rows):
    note(f"vcm gather k={k} s={s} rows={rows}")
    rng = I.stream(51, k, s)
    idx = np.sort(rng.choice(k, s, replace=False)).astype(np.int32)
    idx_d = dev(idx, np.int32)
    bits = I.sign_words(rng, rows, k)
    out = torch.full((rows * ((s + 31) // 32),), -1, dtype=torch.int32, device="cuda")
    fb.fluxbin_vcm_gather(idx_d, s, dev(bits, np.int32), rows, k, fb.DT_BITS, out)
    vals16 = rng.integers(0, 1 << 16, size=(rows, k), dtype=np.uint16)
    out16 = torch.full((rows, s), -1, dtype=torch.int16, device="cuda")
    fb.fluxbin_vcm_gather(idx_d, s, dev(vals16, np.int16), rows, k, fb.DT_F16, out16)
    vals8 = rng.integers(-128, 128, size=(rows, k), dtype=np.int8)
    out8 = torch.full((rows, s), 0, dtype=torch.int8, device="cuda")
    fb.fluxbin_vcm_gather(idx_d, s, dev(vals8, np.int8), rows, k, fb.DT_I8, out8)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32).reshape(rows, -1), orc.vcm_gather_bits(bits, k, idx))
    assert np.array_equal(host_u16(out16), orc.vcm_gather_values(vals16, idx))
    assert np.array_equal(out8.cpu().numpy(), orc.vcm_gather_values(vals8, idx))


# ----------------------------------------------------------------------------- tables

@pytest.mark.parametrize("g,n,k,kb,ks,s,batch", [(4, 64, 512, 2, 0, 0, 1), (4, 70, 300, 2, 1, 37, 3),
                                                (8, 64, 4096, 3, 1, 96, 1), (8, 10, 129, 1, 2, 65, 4)])
def test_build_lut_matches_oracle(fb, orc, g, n, k, kb, ks, s, batch):
    note(f"build_lut g={g} k={k} kb={kb} ks={ks} s={s} batch={batch}")
    layer = I.make_layer(n, k, kb, ks, g, s=s if ks else None, outlier_frac=0.01, seed=(52, g, k))
    x = I.make_x(layer, batch, seed=(52, g, k))
    dl = fb.DeviceLayer(layer, max_batch=batch)
    nf = fb.fluxbin_lut_size(dl.handle, batch)
    lut = torch.full((nf,), float("nan"), dtype=torch.float32, device="cuda")
    fb.fluxbin_build_lut(dl.handle, dev(x, np.int16), batch, lut)
    torch.cuda.synchronize()
    ref, absv = orc.half_luts(layer, x)
    got = lut.cpu().numpy().astype(np.float64).reshape(ref.shape)
    half = 1 << (g - 1)
    tol = (g - 1) * 2.0 ** -24 * np.repeat(absv, half, axis=1)
    assert np.all(np.abs(got - ref) <= tol)
    dl.close()


# ----------------------------------------------------------------------------- exact arithmetic pin

EXACT_CASES = [
    # g, n, k, kb, ks, s, batch
    (4, 512, 512, 2, 0, 0, 1),
    (4, 300, 1000, 2, 1, 77, 1),
    (4, 65, 129, 4, 2, 129, 3),
    (4, 1, 1, 1, 0, 0, 1),
    (4, 130, 4096, 2, 1, 256, 16),
    (8, 200, 4096, 3, 1, 96, 1),
    (8, 64, 257, 1, 2, 31, 4),
]


@pytest.mark.parametrize("g,n,k,kb,ks,s,batch", EXACT_CASES)
def test_gemv_exact_dyadic(fb, orc, g, n, k, kb, ks, s, batch):
    note(f"exact g={g} n={n} k={k} kb={kb} ks={ks} s={s} batch={batch}")
    layer = I.dyadic_layer(n, k, kb, ks, g, s, seed=n + k)
    x = I.dyadic_x(k, batch, seed=k + batch)
    dl = fb.DeviceLayer(layer, max_batch=batch)
    y16 = gemv(fb, dl, x)
    y_ref, _ = orc.gemv_dense(layer, x)
    assert np.array_equal(y16, orc.double_to_half(y_ref)), "y differs from RNE(exact)"
    dl.close()


# ----------------------------------------------------------------------------- the five workloads

def test_workload1_gemv_512(fb, orc):
    note("workload 1: 512x512 kb=2 g=4 batch 1")
    layer = I.workload_layer(1)
    x = I.workload_x(1, layer, 1)
    dl = fb.DeviceLayer(layer)
    y16 = gemv(fb, dl, x)
    r = check_y(orc, layer, x, y16, dl.plan)
    print("ratios (contract, tight):", r)
    dl.close()


def test_workload2_q_proj(fb, orc):
    note("workload 2: q_proj 4096x4096 kb=2 ks=1 s=256 g=4 batch 1")
    layer = I.workload_layer(2)
    assert layer.s == 256 and layer.outliers.size == 41
    # the outlier channels are among the salient columns
    assert set(layer.outliers.tolist()) <= set(layer.sal_idx.tolist())
    x = I.workload_x(2, layer, 1)
    dl = fb.DeviceLayer(layer)
    y16 = gemv(fb, dl, x)
    r = check_y(orc, layer, x, y16, dl.plan)
    print("plan", dl.plan, "ratios (contract, tight):", r)
    dl.close()


@pytest.mark.parametrize("shape_idx", [0, 1, 2, 3])
def test_workload3_llama7b_g8(fb, orc, shape_idx):
    wl = I.WORKLOADS[3]
    for layer_no in (0, wl.layers - 1):
        note(f"workload 3: shape {wl.shapes[shape_idx].name} layer {layer_no}")
        layer = I.workload_layer(3, shape_idx, layer_no)
        x = I.workload_x(3, layer, 1, shape_idx, layer_no)
        dl = fb.DeviceLayer(layer)
        y16 = gemv(fb, dl, x)
        rows = np.unique(np.concatenate([np.arange(64), np.arange(layer.n - 64, layer.n),
                                         I.stream(60, shape_idx, layer_no).choice(layer.n, 512, replace=False)]))
        r = check_y(orc, layer, x, y16, dl.plan, rows=rows)
        print(wl.shapes[shape_idx].name, "plan", dl.plan, "ratios:", r)
        dl.close()


@pytest.mark.parametrize("shape_idx", [0, 1])
def test_workload4_batch_sweep(fb, orc, shape_idx):
    layer = I.workload_layer(4, shape_idx)
    dl = fb.DeviceLayer(layer, max_batch=16)
    ys = {}
    for batch in I.WORKLOADS[4].batches:
        note(f"workload 4: shape {shape_idx} batch {batch}")
        x = I.workload_x(4, layer, batch, shape_idx)
        y16 = gemv(fb, dl, x)
        rows = np.unique(np.concatenate([np.arange(128), I.stream(61, shape_idx, batch).choice(layer.n, 768, replace=False)]))
        r = check_y(orc, layer, x, y16, dl.plan, rows=rows)
        print("batch", batch, "ratios:", r)
        ys[batch] = (x, y16)
    # row b of a batch equals the batch-1 result of that row, bitwise, for the same handle
    x16, y16 = ys[16]
    for b in (0, 7, 15):
        assert np.array_equal(gemv(fb, dl, x16[b:b + 1])[0], y16[b])
    dl.close()


@pytest.mark.parametrize("shape_idx", [0, 1, 2, 3])
def test_workload5_llama70b(fb, orc, shape_idx):
    wl = I.WORKLOADS[5]
    note(f"workload 5: shape {wl.shapes[shape_idx].name} layer 0")
    layer = I.workload_layer(5, shape_idx, 0)
    x = I.workload_x(5, layer, 1, shape_idx, 0)
    dl = fb.DeviceLayer(layer)
    y16 = gemv(fb, dl, x)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(layer.n - 64, layer.n),
                                     I.stream(62, shape_idx).choice(layer.n, 384, replace=False)]))
    r = check_y(orc, layer, x, y16, dl.plan, rows=rows)
    print(wl.shapes[shape_idx].name, "plan", dl.plan, "ratios:", r)
    dl.close()


# ----------------------------------------------------------------------------- edge cases

EDGE = [
    # g, n, k, kb, ks, s, batch, cpb, waves
    (4, 1, 1, 1, 0, 0, 1, 0, 0),
    (4, 63, 5, 1, 1, 1, 1, 0, 0),
    (4, 65, 127, 3, 2, 127, 2, 0, 0),
    (4, 2000, 33, 2, 1, 33, 5, 0, 0),
    (4, 777, 1031, 4, 2, 500, 16, 0, 0),
    (4, 4096, 4096, 2, 1, 256, 1, 1, 0),
    (4, 4096, 4096, 2, 1, 256, 1, 2, 0),
    (4, 4096, 4096, 2, 1, 256, 1, 4, 0),
    (4, 4096, 4096, 2, 1, 256, 1, 8, 0),
    (4, 4096, 4096, 2, 1, 256, 1, 2, 8),
    (4, 1000, 4096, 2, 1, 96, 3, 4, 8),
    (4, 577, 300, 1, 1, 40, 1, 1, 4),
    (4, 257, 11008, 2, 1, 224, 8, 2, 0),
    (4, 257, 11008, 2, 1, 224, 8, 3, 8),
    # long workgroup ranges (8-deep prefetch): segment changes inside a range,
    # a last range shorter than the prefetch depth, the largest range
    (4, 4096, 4096, 2, 1, 256, 1, 16, 4),
    (4, 300, 4096, 4, 2, 1000, 1, 20, 8),
    (4, 300, 4096, 4, 2, 1000, 1, 31, 8),
    (4, 130, 2500, 3, 1, 700, 2, 9, 8),
    (8, 1, 8, 1, 0, 0, 1, 0, 0),
    (8, 100, 1000, 4, 2, 999, 3, 0, 0),
    (8, 4096, 4096, 3, 1, 96, 1, 1, 0),
    (8, 4096, 4096, 3, 1, 96, 1, 4, 0),
    (8, 4096, 4096, 3, 1, 96, 2, 2, 8),
]


@pytest.mark.parametrize("g,n,k,kb,ks,s,batch,cpb,waves", EDGE)
def test_gemv_edge_cases(fb, orc, g, n, k, kb, ks, s, batch, cpb, waves):
    note(f"edge g={g} n={n} k={k} kb={kb} ks={ks} s={s} batch={batch} cpb={cpb} waves={waves}")
    layer = I.make_layer(n, k, kb, ks, g, s=s if ks else None, outlier_frac=0.01, seed=(63, n, k))
    x = I.make_x(layer, batch, seed=(63, n, k))
    dl = fb.DeviceLayer(layer, max_batch=batch, chunks_per_block=cpb, waves_per_block=waves)
    if waves:
        assert dl.plan["rows_per_block"] == 64 * waves
    y16 = gemv(fb, dl, x)
    rows = None if n <= 4096 else I.stream(64, n).choice(n, 1024, replace=False)
    check_y(orc, layer, x, y16, dl.plan, rows=rows)
    dl.close()


# Two or four waves per row tile (g = 4, one batch row, automatic plan of a layer whose ranges
# would be 2 chunks long over more than 256 workgroups): each wave of a tile takes one part of a
# 4- or 8-chunk range and the others hand their partials to the first through LDS.  q_proj and
# the 7B up and down shapes; rows that fill neither the last tile nor the last row block (2100:
# one tile of the last block, 4097: one row of it); 1-chunk salient ranges (all but one wave of a
# tile look up nothing), 2- and 3-chunk ones (1 + 1, 1 + 2; at four waves 0 + 1 + 1 + 1); global
# segments cut into ranges of 3 and 4, a last chunk of 104 columns (k = 1000), of 32 (k = 4000) or
# of one (k = 129, whose 2-chunk segments make 1 + 1 ranges throughout); three and four global and
# two salient bases.  Dyadic inputs must give RNE(exact) bitwise; random ones the rounding bound.
SEVERAL_WAVES = [
    # n, k, kb, ks, s, waves per row tile
    (4096, 4096, 2, 1, 256, 4),
    (4097, 4096, 2, 1, 256, 4),
    (4000, 4000, 2, 1, 100, 4),
    (3000, 4096, 3, 2, 300, 4),
    (5000, 3000, 3, 2, 300, 4),
    (2100, 4096, 2, 1, 100, 2),
    (9000, 1000, 2, 1, 300, 2),
    (4096, 11008, 2, 1, 224, 2),
    (11008, 4096, 2, 1, 96, 2),
    (4097, 11008, 2, 1, 224, 2),
    (16000, 129, 4, 2, 100, 2),
]


@pytest.mark.parametrize("n,k,kb,ks,s,wpt", SEVERAL_WAVES)
def test_several_waves_per_row_tile(fb, orc, n, k, kb, ks, s, wpt):
    note(f"{wpt} waves per tile n={n} k={k} kb={kb} ks={ks} s={s}")
    layer = I.dyadic_layer(n, k, kb, ks, 4, s, seed=n + k + 7)
    x = I.dyadic_x(k, 1, seed=k + 7)
    dl = fb.DeviceLayer(layer, max_batch=1)
    assert dl.plan["threads_per_block"] == wpt * dl.plan["rows_per_block"] == 512, dl.plan
    y16 = gemv(fb, dl, x)
    y_ref, _ = orc.gemv_dense(layer, x)
    assert np.array_equal(y16, orc.double_to_half(y_ref)), "y differs from RNE(exact)"
    dl.close()
    layer = I.make_layer(n, k, kb, ks, 4, s=s if ks else None, outlier_frac=0.01, seed=(65, n, k))
    x = I.make_x(layer, 1, seed=(65, n, k))
    dl = fb.DeviceLayer(layer, max_batch=1)
    assert dl.plan["threads_per_block"] == wpt * dl.plan["rows_per_block"]
    y16 = gemv(fb, dl, x)
    rows = None if n <= 4096 else I.stream(65, n).choice(n, 1024, replace=False)
    check_y(orc, layer, x, y16, dl.plan, rows=rows)
    dl.close()


# g = 8 bank-private tables (one batch row, per-row scales, fp32 entries): regions of 2 and 4 chunks
# at 4 and 8 waves, column ranges shorter than the region (k = 1000: 8 chunks cut 3-3-2; k = 384: one
# range of 3), rows that fill neither the last tile nor the last row block, a single row, salient
# segments of 1 and 2 chunks, a given 4-chunk range at the automatic wave count (one 4-chunk region,
# 16-wave workgroups of 1024 rows: 1100 rows fill one block and two tiles of the next, the last
# tile partly), and the automatic plan (2-chunk regions, two in turn per range for the wide
# layers: k = 11008 cuts 86 chunks into ranges of 3 and 4, so some ranges end inside their second
# region, and its 2-chunk salient ranges have no second region).  Dyadic inputs must give
# RNE(exact) bitwise; random inputs the rounding bound.
BANKED = [
    # n, k, kb, ks, s, cpb, waves, region
    (4000, 1000, 3, 1, 200, 4, 8, 4),
    (4000, 1000, 3, 1, 200, 3, 4, 4),
    (4000, 1000, 3, 1, 200, 2, 8, 2),
    (4000, 1000, 3, 1, 200, 2, 4, 2),
    (4000, 1000, 3, 1, 200, 1, 8, 2),
    (100, 11008, 3, 1, 220, 4, 8, 4),
    (100, 11008, 3, 1, 220, 2, 4, 2),
    (600, 384, 2, 2, 129, 4, 8, 4),
    (600, 384, 2, 2, 129, 2, 8, 2),
    (1, 4096, 1, 0, 0, 4, 8, 4),
    (1, 4096, 1, 0, 0, 2, 4, 2),
    (513, 4096, 4, 2, 82, 0, 0, None),
    (1100, 11008, 3, 1, 220, 4, 0, 4),
    (300, 11008, 3, 1, 220, 0, 0, None),
    (1100, 11008, 3, 1, 220, 0, 0, None),
]


@pytest.mark.parametrize("n,k,kb,ks,s,cpb,waves,region", BANKED)
def test_g8_banked_tables(fb, orc, n, k, kb, ks, s, cpb, waves, region):
    note(f"banked g=8 n={n} k={k} kb={kb} ks={ks} s={s} cpb={cpb} waves={waves}")
    layer = I.dyadic_layer(n, k, kb, ks, 8, s, seed=n + 3 * k + cpb)
    x = I.dyadic_x(k, 1, seed=k + cpb)
    dl = fb.DeviceLayer(layer, chunks_per_block=cpb, waves_per_block=waves)
    # automatic plan: 2-chunk regions, one or two per range
    assert dl.plan["banked_tables"] == (region or 2)
    assert dl.plan["table_chunks"] == dl.plan["banked_tables"]
    if not waves:  # automatic wave count: 16 for 4-chunk regions, 8 for 2-chunk ones
        assert dl.plan["rows_per_block"] == (1024 if dl.plan["banked_tables"] == 4 else 512)
    y16 = gemv(fb, dl, x)
    y_ref, _ = orc.gemv_dense(layer, x)
    assert np.array_equal(y16, orc.double_to_half(y_ref)), "y differs from RNE(exact)"
    dl.close()
    layer = I.make_layer(n, k, kb, ks, 8, s=s if ks else None, outlier_frac=0.01, seed=(65, n, k))
    x = I.make_x(layer, 1, seed=(65, n, k))
    dl = fb.DeviceLayer(layer, chunks_per_block=cpb, waves_per_block=waves)
    y16 = gemv(fb, dl, x)
    check_y(orc, layer, x, y16, dl.plan)
    dl.close()


# The split reduction at its limit: one-chunk column ranges cut these rows into exactly 255
# ranges, the most the 8-bit arrival count of a reduction word takes (the last arriver finds 254
# arrivals before its own); g = 4 with and without a salient basis (ragged k and s), and the
# bank-private g = 8 kernel.  Dyadic inputs must give RNE(exact) bitwise; random inputs the bound.
SPLIT_LIMIT = [
    # n, k, kb, ks, s, g
    (300, 10800, 3, 0, 0, 4),
    (257, 16100, 2, 1, 384, 4),
    (300, 10800, 3, 0, 0, 8),
]


@pytest.mark.parametrize("n,k,kb,ks,s,g", SPLIT_LIMIT)
def test_split_count_at_its_limit(fb, orc, n, k, kb, ks, s, g):
    note(f"255 splits: n={n} k={k} kb={kb} ks={ks} s={s} g={g}")
    layer = I.dyadic_layer(n, k, kb, ks, g, s, seed=n + k + g)
    x = I.dyadic_x(k, 1, seed=k + g)
    dl = fb.DeviceLayer(layer, chunks_per_block=1)
    assert dl.plan["splits"] == 255 and dl.plan["chunks_per_block"] == 1
    y16 = gemv(fb, dl, x)
    y_ref, _ = orc.gemv_dense(layer, x)
    assert np.array_equal(y16, orc.double_to_half(y_ref)), "y differs from RNE(exact)"
    dl.close()
    layer = I.make_layer(n, k, kb, ks, g, s=s if ks else None, outlier_frac=0.01, seed=(66, n, k))
    x = I.make_x(layer, 1, seed=(66, n, k))
    dl = fb.DeviceLayer(layer, chunks_per_block=1)
    y16 = gemv(fb, dl, x)
    check_y(orc, layer, x, y16, dl.plan)
    dl.close()


def test_batch_zero_is_a_no_op(fb):
    layer = I.workload_layer(1)
    dl = fb.DeviceLayer(layer)
    y = torch.full((1, layer.n), 1234, dtype=torch.int16, device="cuda")
    x = torch.zeros((1, layer.k), dtype=torch.int16, device="cuda")
    fb.fluxbin_gemv(dl.handle, x, y, 0)
    torch.cuda.synchronize()
    assert bool((y == 1234).all())
    dl.close()


# ----------------------------------------------------------------------------- determinism, batch, graphs

def test_repeat_calls_are_bitwise_identical(fb):
    note("determinism: 20 calls of workload 2")
    layer = I.workload_layer(2)
    x = dev(I.workload_x(2, layer, 1), np.int16)
    dl = fb.DeviceLayer(layer)
    assert dl.plan["splits"] > 1  # exercises the cross-workgroup reduction
    y0 = torch.empty((1, layer.n), dtype=torch.int16, device="cuda")
    dl.gemv(x, y0)
    y = torch.empty_like(y0)
    for _ in range(20):
        dl.gemv(x, y)
        torch.cuda.synchronize()
        assert torch.equal(y, y0)
    dl.close()


def test_graph_capture_replays_match_eager(fb):
    note("graph capture: 4 GEMVs of workload 2 shape, 3 replays")
    layer = I.workload_layer(2)
    dls = [fb.DeviceLayer(layer) for _ in range(2)]
    xs = [dev(I.workload_x(2, layer, 1, layer=i), np.int16) for i in range(4)]
    eager = []
    for i, x in enumerate(xs):
        y = torch.empty((1, layer.n), dtype=torch.int16, device="cuda")
        dls[i % 2].gemv(x, y)
        eager.append(y)
    torch.cuda.synchronize()
    outs = [torch.zeros((1, layer.n), dtype=torch.int16, device="cuda") for _ in xs]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i, x in enumerate(xs):
                dls[i % 2].gemv(x, outs[i], stream=s)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        for o in outs:
            o.zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), f"replay {rep} differs"
        del junk
    for d in dls:
        d.close()


# ----------------------------------------------------------------------------- error paths

def test_injected_launch_fault_leaves_output_untouched(fb, monkeypatch):
    layer = I.workload_layer(1)
    monkeypatch.setenv("FLUXBIN_FAULT", "launch")
    dl = fb.DeviceLayer(layer)
    monkeypatch.delenv("FLUXBIN_FAULT")
    y = torch.full((1, layer.n), 77, dtype=torch.int16, device="cuda")
    x = torch.zeros((1, layer.k), dtype=torch.int16, device="cuda")
    with pytest.raises(fb.FluxbinError) as ei:
        fb.fluxbin_gemv(dl.handle, x, y, 1)
    assert ei.value.status == fb.ERR_HIP
    lut = torch.full((16,), 5.0, device="cuda")
    with pytest.raises(fb.FluxbinError):
        fb.fluxbin_build_lut(dl.handle, x, 1, lut)
    torch.cuda.synchronize()
    assert bool((y == 77).all()) and bool((lut == 5.0).all())
    dl.close()


@pytest.mark.parametrize("bad", ["unsorted", "duplicate", "out_of_range", "negative"])
def test_create_rejects_bad_salient_index(fb, bad):
    layer = I.make_layer(128, 256, 1, 1, 4, s=8, seed=(65, 0, 0))
    idx = layer.sal_idx.copy()
    if bad == "unsorted":
        idx[[2, 3]] = idx[[3, 2]]
    elif bad == "duplicate":
        idx[4] = idx[3]
    elif bad == "out_of_range":
        idx[-1] = layer.k
    else:
        idx[0] = -1
    layer.sal_idx = idx
    with pytest.raises(fb.FluxbinError) as ei:
        fb.DeviceLayer(layer)
    assert ei.value.status == fb.ERR_INVALID_ARGUMENT


def test_create_rejects_small_workspace_and_gemv_rejects_big_batch(fb):
    layer = I.workload_layer(2)
    dl = fb.DeviceLayer(layer)
    d = dl.make_desc()
    d.workspace = fb._ptr(dl.workspace)
    d.workspace_bytes = fb.fluxbin_workspace_size(d) - 1
    with pytest.raises(fb.FluxbinError) as ei:
        fb.fluxbin_create(d)
    assert ei.value.status == fb.ERR_WORKSPACE
    x = torch.zeros((2, layer.k), dtype=torch.int16, device="cuda")
    y = torch.zeros((2, layer.n), dtype=torch.int16, device="cuda")
    with pytest.raises(fb.FluxbinError) as ei:
        fb.fluxbin_gemv(dl.handle, x, y, 2)
    assert ei.value.status == fb.ERR_INVALID_ARGUMENT
    dl.close()


# ----------------------------------------------------------------------------- dense context kernel

@pytest.mark.parametrize("n,k,batch", [(4096, 4096, 1), (300, 1000, 3), (64, 8, 16)])
def test_dense_f16_context_kernel(fb, orc, n, k, batch):
    note(f"dense fp16 n={n} k={k} batch={batch}")
    rng = np.random.default_rng(n + k)
    w = rng.normal(0, 0.02, (n, k)).astype(np.float16).view(np.uint16)
    x = rng.normal(0, 1, (batch, k)).astype(np.float16).view(np.uint16)
    y = torch.empty((batch, n), dtype=torch.int16, device="cuda")
    fb.fluxbin_dense_gemv_f16(dev(w, np.int16), n, k, dev(x, np.int16), y, batch)
    torch.cuda.synchronize()
    y_ref, mag = orc.dense_f16_gemv(w, x)
    got = orc.half_to_double(host_u16(y))
    assert np.all(np.abs(got - y_ref) <= 2.0 ** -11 * np.abs(y_ref) + 2.0 ** -24 * (k + 8) * mag + 2.0 ** -25)
