"""GPU tests of the boundary's own guarantees, through the C ABI.

  * the split reduction never returns a silently wrong number: a row whose
    partial sum over one column range is outside the fixed-point range is
    written as NaN, every other row is exact;
  * fluxbin_reset_workspace restores dirty reduction words (eagerly and inside
    a captured graph);
  * row-major sign words and block-wise scales handed to fluxbin_create give
    bitwise the result of the tiled ones;
  * the measurement kernels run.
"""
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


@pytest.fixture(scope="module")
def orc():
    from oracle import oracle
    return oracle


def note(msg):
    print(f"[case] {msg}", flush=True)


def dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a).view(dtype)).cuda()


def run(fb, dl, x_np):
    x = dev(x_np, np.int16)
    y = torch.full((x_np.shape[0], dl.layer.n), 0x1234, dtype=torch.int16, device="cuda")
    dl.gemv(x, y)
    torch.cuda.synchronize()
    return y.cpu().numpy().view(np.uint16)


def h16(v):
    return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def test_partials_beyond_the_fixed_point_range_give_nan_not_a_wrong_number(fb, orc):
    # two identical global bases.  Rows 0..63: all signs +1, row scales +1 and -1, so the row total
    # is exactly 0 (well inside fp16), but with x = 256 and c = 8 every 256-column range sums to
    # +-2^19 >= 2^17: NaN.  The other rows: random signs, both row scales 2^-6, so partials stay
    # below 2^13, every value is an exact multiple of 2^5, and y must be the oracle's exactly.
    note("reduction overflow: 256 x 4096, kb 2 with cancelling bases")
    n, k = 256, 4096
    layer = I.make_layer(n, k, 2, 0, 4, seed=(71, 0, 0))
    bits = layer.bits_g.copy()
    bits[0, :64, :] = 0xFFFFFFFF
    bits[1] = bits[0]
    layer.bits_g = bits
    layer.c_g = np.full((2, k), 8.0, np.float64).astype(np.float16).view(np.uint16)
    r = np.full(n, 2.0 ** -6)
    r[:64] = 1.0
    sgn = np.ones(n)
    sgn[:64] = -1.0
    layer.r_g = np.stack([h16(r), h16(sgn * r)])
    x = np.full((1, k), 256.0).astype(np.float16).view(np.uint16)
    dl = fb.DeviceLayer(layer, chunks_per_block=2)
    assert dl.plan["splits"] == 2 * 16
    y = run(fb, dl, x)
    yd = orc.half_to_double(y)[0]
    assert np.all(np.isnan(yd[:64])), yd[:64]
    y_ref, _ = orc.gemv_dense(layer, x, rows=np.arange(64, n))
    assert np.any(y_ref != 0)
    assert np.array_equal(y[0, 64:], orc.double_to_half(y_ref)[0]), (yd[64:][:8], y_ref[0][:8])
    # the words are clean again after the flagged call: an ordinary call is exact
    layer2 = I.dyadic_layer(n, k, 2, 0, 4, 0, seed=72)
    dl2 = fb.DeviceLayer(layer2, chunks_per_block=2)
    x2 = I.dyadic_x(k, 1, seed=72)
    y2 = run(fb, dl2, x2)
    y_ref2, _ = orc.gemv_dense(layer2, x2)
    assert np.array_equal(y2, orc.double_to_half(y_ref2))
    # and the overflowing handle, called again, flags the same rows and nothing else
    y = run(fb, dl, x)
    assert np.all(np.isnan(orc.half_to_double(y)[0, :64])) and not np.any(np.isnan(orc.half_to_double(y)[0, 64:]))
    dl.close()
    dl2.close()


def test_reset_workspace_restores_dirty_reduction_words(fb):
    note("workspace reset: workload 2, dirty words")
    layer = I.workload_layer(2)
    x = dev(I.workload_x(2, layer, 1), np.int16)
    dl = fb.DeviceLayer(layer)
    assert dl.plan["splits"] > 1 and dl.workspace is not None
    y0 = torch.empty((1, layer.n), dtype=torch.int16, device="cuda")
    dl.gemv(x, y0)
    torch.cuda.synchronize()
    # words left behind by a call that did not complete: nonzero counts and values
    dl.workspace.fill_(0x5A)
    y = torch.empty_like(y0)
    dl.gemv(x, y)  # reads the dirty words: its result is garbage (not checked) and the words stay dirty
    dl.reset_workspace()
    dl.gemv(x, y)
    torch.cuda.synchronize()
    assert torch.equal(y, y0)
    # the reset captured in a graph ahead of the call, replayed after more dirt
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    out = torch.zeros_like(y0)
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            dl.reset_workspace(stream=s)
            dl.gemv(x, out, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        dl.workspace.fill_(0x33 + rep)
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, y0), f"replay {rep}"
    dl.close()


@pytest.mark.parametrize("kind", ["per_row_q_proj", "per_row_g8", "block_wise_s8", "block_wise_s16_g8"])
def test_row_major_inputs_match_tiled_inputs_bitwise(fb, kind):
    note(f"row-major inputs: {kind}")
    if kind == "per_row_q_proj":
        layer = I.workload_layer(2)
        x = I.workload_x(2, layer, 2)
    elif kind == "per_row_g8":
        layer = I.make_layer(300, 1000, 3, 1, 8, s=40, seed=(73, 0, 0))
        x = I.make_x(layer, 2, seed=(73, 0, 0))
    elif kind == "block_wise_s8":
        layer = I.make_grouped_layer(1000, 1100, 2, 2, 4, 128, 8, seed=(74, 0, 0))
        x = I.make_x(layer, 2, seed=(74, 0, 0))
    else:
        layer = I.make_grouped_layer(700, 2048, 2, 1, 8, 128, 16, seed=(75, 0, 0))
        x = I.make_x(layer, 2, seed=(75, 0, 0))
    ys = []
    for layout in (fb.LAYOUT_TILED, fb.LAYOUT_ROWMAJOR):
        dl = fb.DeviceLayer(layer, max_batch=2, layout=layout)
        ys.append(run(fb, dl, x))
        dl.close()
    assert np.array_equal(ys[0], ys[1])


def test_timed_gemv_matches_the_plain_call(fb):
    note("timed gemv: workload 2 and a 2-group batch")
    for layer, batch, mb in ((I.workload_layer(2), 1, 1), (I.make_layer(300, 700, 2, 1, 4, s=40, seed=(76, 0, 0)), 20, 20)):
        x = dev(I.make_x(layer, batch, seed=(76, 1, 0)), np.int16)
        dl = fb.DeviceLayer(layer, max_batch=mb)
        y0 = torch.empty((batch, layer.n), dtype=torch.int16, device="cuda")
        dl.gemv(x, y0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        e1.record()  # creates the events
        y = torch.zeros_like(y0)
        fb.fluxbin_gemv_timed(dl.handle, x, y, batch, e0, e1)
        torch.cuda.synchronize()
        assert torch.equal(y, y0)
        assert e0.elapsed_time(e1) > 0
        dl.close()


def test_measurement_kernels_run(fb):
    note("probes: stream read, empty kernel, table lookups")
    buf = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(256 * 256, dtype=torch.int32, device="cuda")
    for depth in (1, 4, 16):
        fb.fluxbin_probe_stream_read(buf, buf.numel(), depth, 256, 0x9E3779B9, sink)  # the XOR of zeros is 0
    fb.fluxbin_probe_empty(1024, 256)
    fs = torch.zeros(64 * 256, dtype=torch.float32, device="cuda")
    for g, nb in ((4, 1), (4, 4), (4, 16), (8, 1), (8, 4)):
        fb.fluxbin_probe_lds_lookup(g, nb, 64, 4, -1.0, fs)  # table entries are >= 0 and sums finite: never -1
    fb2 = torch.zeros(64 * 512, dtype=torch.float32, device="cuda")
    for region in (2, 4):
        fb.fluxbin_probe_lds_lookup_banked(region, 64, 4, -1.0, fb2)
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0 and float(fs.abs().sum()) == 0.0 and float(fb2.abs().sum()) == 0.0
