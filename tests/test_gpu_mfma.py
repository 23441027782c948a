"""GPU parity of the matrix-core route (FLUXBIN_COMPUTE_MFMA) against the fp64 oracle.

The route computes the same layer product as the LUT GEMV (FluxBin summary, section 3
"Quantization", "Salient-Aware Hybrid Bases", "Virtual Columnar Mapping"), as a dense contraction
for prefill batches.  Bars:
  * dyadic inputs (every product and partial sum exact in fp32): y equals RNE-to-fp16 of the exact
    value, per-row and block-wise scales, ragged shapes (rows, columns, batch, |S|);
  * the workload shapes: the contract |y - y_ref| <= 1e-3 * sum_j |W_hat_ij x_j| per row and the
    first-order fp32 bound with one rounding per accumulated column (the matrix core adds 16
    exact products per step);
  * batch independence: every row of a batch equals, bitwise, the same row run alone (the kernel
    instance changes with the batch width, the per-element arithmetic does not);
  * repeated calls are bitwise identical.
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


def mfma_layer(fb, layer, batch, cpb=0):
    return fb.DeviceLayer(layer, max_batch=batch, chunks_per_block=cpb, compute=fb.COMPUTE_MFMA)


def mfma_steps(layer, plan):
    return max(layer.k, layer.s) + layer.kb + layer.ks + plan["splits"] + 3


EXACT = [
    # n, k, kb, ks, s, batch, cpb
    (130, 1000, 2, 1, 77, 40, 0),      # k % 8 != 0: element-wise staging; ragged rows and columns
    (64, 257, 1, 2, 31, 10, 0),
    (65, 129, 4, 2, 129, 128, 0),
    (300, 4096, 2, 1, 256, 1, 0),
    (300, 4096, 2, 1, 256, 33, 3),
    (1, 128, 1, 0, 0, 1, 0),           # one row, one chunk, no split
    (128, 4096, 1, 0, 0, 64, 32),      # one range per row: direct stores
    (4096, 1024, 2, 2, 100, 97, 1),
]


@pytest.mark.parametrize("n,k,kb,ks,s,batch,cpb", EXACT)
def test_mfma_exact_dyadic(fb, orc, n, k, kb, ks, s, batch, cpb):
    note(f"mfma exact n={n} k={k} kb={kb} ks={ks} s={s} batch={batch} cpb={cpb}")
    layer = I.dyadic_layer(n, k, kb, ks, 4, s, seed=n + k + batch)
    x = I.dyadic_x(k, batch, seed=k + batch + 5)
    dl = mfma_layer(fb, layer, batch, cpb)
    y16 = gemv(fb, dl, x)
    y_ref, _ = orc.gemv_dense(layer, x)
    assert np.array_equal(y16, orc.double_to_half(y_ref)), "y differs from RNE(exact)"
    dl.close()


GROUPED_EXACT = [
    # n, k, kb, ks, sal_group, batch, cpb
    (300, 1000, 2, 2, 8, 5, 0),
    (130, 4096, 2, 2, 8, 64, 0),
    (65, 136, 4, 2, 8, 3, 0),
    (64, 512, 2, 1, 16, 100, 0),
    (200, 4096, 3, 1, 16, 1, 5),
    (1, 128, 1, 0, 0, 1, 0),
    (777, 2048, 2, 2, 16, 128, 2),
]


@pytest.mark.parametrize("n,k,kb,ks,sg,batch,cpb", GROUPED_EXACT)
def test_mfma_grouped_exact_dyadic(fb, orc, n, k, kb, ks, sg, batch, cpb):
    note(f"mfma block-wise exact n={n} k={k} kb={kb} ks={ks} sal_group={sg} batch={batch} cpb={cpb}")
    layer = I.dyadic_grouped_layer(n, k, kb, ks, 4, 128, sg or 8, seed=n + k + 3)
    x = I.dyadic_x(k, batch, seed=k + batch + 6)
    dl = mfma_layer(fb, layer, batch, cpb)
    y16 = gemv(fb, dl, x)
    y_ref, _ = orc.gemv_dense(layer, x)
    assert np.array_equal(y16, orc.double_to_half(y_ref)), "y differs from RNE(exact)"
    dl.close()


SHAPES = [
    # name, k, n, kb, ks, s (per-row) or sal_group (block-wise), batch, blockwise
    ("mlp_up_b128", 4096, 11008, 2, 1, 96, 128, False),
    ("mlp_down_b64", 11008, 4096, 2, 1, 224, 64, False),
    ("q_proj_b33", 4096, 4096, 2, 1, 256, 33, False),
    ("q_proj_b1", 4096, 4096, 2, 1, 256, 1, False),
    ("q_proj_s8_b100", 4096, 4096, 2, 2, 8, 100, True),
    ("q_proj_s16_b32", 4096, 4096, 2, 2, 16, 32, True),
    ("70b_down_s8_b16", 28672, 8192, 2, 2, 8, 16, True),
]


@pytest.mark.parametrize("name,k,n,kb,ks,s,batch,blockwise", SHAPES)
def test_mfma_shapes(fb, orc, name, k, n, kb, ks, s, batch, blockwise):
    note(f"mfma shape {name}: k={k} n={n} kb={kb} ks={ks} batch={batch}")
    if blockwise:
        layer = I.make_grouped_layer(n, k, kb, ks, 4, 128, s, outlier_frac=0.01, seed=(98, n, k))
    else:
        layer = I.make_layer(n, k, kb, ks, 4, s=s, outlier_frac=0.01, seed=(98, n, k))
    x = I.make_x(layer, batch, seed=(98, n, k))
    dl = mfma_layer(fb, layer, batch)
    y16 = gemv(fb, dl, x)
    rows = np.unique(np.concatenate([np.arange(32), np.arange(n - 32, n),
                                     I.stream(99, n, batch).choice(n, 160, replace=False)]))
    r = check_y(orc, layer, x, y16, dl.plan, rows=rows, steps=mfma_steps(layer, dl.plan))
    print(name, "plan", dl.plan, "ratios (contract, tight):", r)
    for b in sorted({0, batch // 2, batch - 1}):
        assert np.array_equal(gemv(fb, dl, x[b:b + 1])[0], y16[b]), f"batch row {b} depends on the batch"
    assert np.array_equal(gemv(fb, dl, x), y16), "repeat call differs"
    dl.close()


def test_mfma_and_lut_routes_agree_within_the_contract(fb, orc):
    n, k, batch = 1000, 2048, 24
    note(f"mfma vs lut n={n} k={k} batch={batch}")
    layer = I.make_layer(n, k, 2, 1, 4, s=64, outlier_frac=0.01, seed=(100, n, k))
    x = I.make_x(layer, batch, seed=(100, n, k))
    a = mfma_layer(fb, layer, batch)
    b = fb.DeviceLayer(layer, max_batch=batch)
    ya, yb = gemv(fb, a, x), gemv(fb, b, x)
    check_y(orc, layer, x, ya, a.plan, steps=mfma_steps(layer, a.plan))
    check_y(orc, layer, x, yb, b.plan)
    a.close()
    b.close()


def test_mfma_graph_capture_replays_match_eager(fb):
    """The route's two launches (multiply, then the sum of the ranges' partials) captured in a
    HIP graph: every replay, with eager work in between, equals the eager result."""
    n, k, batch = 2000, 4096, 48
    note(f"mfma graph capture n={n} k={k} batch={batch}")
    layer = I.make_layer(n, k, 2, 1, 4, s=128, outlier_frac=0.01, seed=(101, n, k))
    x = torch.from_numpy(I.make_x(layer, batch, seed=(101, n, k)).view(np.int16)).cuda()
    dl = mfma_layer(fb, layer, batch)
    assert dl.plan["splits"] > 1
    eager = torch.empty((batch, n), dtype=torch.int16, device="cuda")
    dl.gemv(x, eager)
    torch.cuda.synchronize()
    out = torch.zeros((batch, n), dtype=torch.int16, device="cuda")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            dl.gemv(x, out, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        out.zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs"
        del junk
    dl.close()


def test_mfma_rejects_on_the_host(fb):
    layer = I.make_layer(256, 512, 1, 0, 4, seed=(102, 0, 0))
    with pytest.raises(fb.FluxbinError):
        fb.DeviceLayer(layer, max_batch=8, waves_per_block=8, compute=fb.COMPUTE_MFMA)
    dl = mfma_layer(fb, layer, 8)
    x = torch.zeros((9, 512), dtype=torch.int16, device="cuda")
    y = torch.zeros((9, 256), dtype=torch.int16, device="cuda")
    with pytest.raises(fb.FluxbinError):
        dl.gemv(x, y)  # batch above max_batch
    dl.close()


@pytest.mark.parametrize("compute", ["lut", "mfma"])
def test_unaligned_x_gives_the_same_result(fb, orc, compute):
    """x starting 2 bytes past a 16-byte boundary: the matrix-core route stages it element by
    element (no 16-byte loads); both routes give the bits of the aligned call."""
    n, k, batch = 300, 1024, 20
    note(f"unaligned x, {compute}: n={n} k={k} batch={batch}")
    layer = I.make_layer(n, k, 2, 1, 4, s=64, outlier_frac=0.01, seed=(103, n, k))
    x_np = I.make_x(layer, batch, seed=(103, n, k))
    route = fb.COMPUTE_MFMA if compute == "mfma" else fb.COMPUTE_LUT
    dl = fb.DeviceLayer(layer, max_batch=batch, compute=route)
    base = torch.zeros(batch * k + 8, dtype=torch.int16, device="cuda")
    xa = base[:batch * k].view(batch, k)
    xu = base[1:1 + batch * k].view(batch, k)
    assert xu.data_ptr() % 16 == 2
    xa.copy_(torch.from_numpy(x_np.view(np.int16)))
    ya = torch.zeros((batch, n), dtype=torch.int16, device="cuda")
    dl.gemv(xa, ya)
    torch.cuda.synchronize()
    xu.copy_(torch.from_numpy(x_np.view(np.int16)))
    yu = torch.zeros((batch, n), dtype=torch.int16, device="cuda")
    dl.gemv(xu, yu)
    torch.cuda.synchronize()
    assert torch.equal(ya, yu)
    check_y(orc, layer, x_np, yu.cpu().numpy().view(np.uint16), dl.plan,
            steps=mfma_steps(layer, dl.plan) if compute == "mfma" else None)
    dl.close()
