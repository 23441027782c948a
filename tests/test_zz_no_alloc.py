"""fluxbin_gemv_static, the entry point for callers that cannot allocate: its split-reduction words live
in the library's static device array instead of a workspace.  Checked through the C ABI against
fluxbin_gemv on the same handle (the same kernels and arithmetic: bitwise equal y), on consecutive calls
of different sizes, on a handle created without any workspace, under graph capture, and at its size
limit.
"""
import ctypes

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


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def both(fb, dl, x, batch):
    """y from fluxbin_gemv and from fluxbin_gemv_static on the same handle."""
    y0 = torch.full((batch, dl.layer.n), 0x1111, dtype=torch.int16, device="cuda")
    y1 = torch.full((batch, dl.layer.n), 0x2222, dtype=torch.int16, device="cuda")
    fb.fluxbin_gemv(dl.handle, x, y0, batch)
    fb.fluxbin_gemv_static(dl.handle, x, y1, batch)
    torch.cuda.synchronize()
    return y0, y1


def test_static_scratch_matches_the_workspace_call_on_consecutive_calls(fb):
    note("static scratch: q_proj at batch 4, then a 512 x 512 layer at batch 1, then q_proj again")
    big = I.workload_layer(2)
    dl_big = fb.DeviceLayer(big, max_batch=4)
    assert dl_big.plan["splits"] > 1
    x_big = dev(I.workload_x(2, big, 4))
    y_first, y1 = both(fb, dl_big, x_big, 4)
    assert torch.equal(y_first, y1)
    # a second, smaller call: fewer words than the first one left behind
    small = I.make_layer(512, 512, 2, 1, 4, s=64, outlier_frac=0.01, seed=(77, 0, 0))
    dl_small = fb.DeviceLayer(small, max_batch=1, chunks_per_block=1)
    assert dl_small.plan["splits"] > 1
    x_small = dev(I.make_x(small, 1, seed=(77, 0, 0)))
    y0, y1 = both(fb, dl_small, x_small, 1)
    assert torch.equal(y0, y1)
    # and the first shape again
    y0b, y1b = both(fb, dl_big, x_big, 4)
    assert torch.equal(y0b, y1b) and torch.equal(y0b, y_first)
    dl_big.close()
    dl_small.close()


def test_static_scratch_with_the_banked_g8_kernel(fb):
    note("static scratch: g = 8 banked plans, two 2-chunk regions per range and one")
    for n, k in ((300, 11008), (700, 1024)):
        layer = I.make_layer(n, k, 3, 1, 8, s=224 if k > 4096 else 32, outlier_frac=0.0, seed=(78, n, k))
        dl = fb.DeviceLayer(layer)
        assert dl.plan["banked_tables"] == 2 and dl.plan["splits"] > 1
        assert dl.plan["chunks_per_block"] == (4 if k > 4096 else 2)
        x = dev(I.make_x(layer, 1, seed=(78, n, k)))
        y0, y1 = both(fb, dl, x, 1)
        assert torch.equal(y0, y1)
        dl.close()


def test_handle_without_workspace(fb):
    note("static scratch: q_proj handle created without a workspace")
    layer = I.workload_layer(2)
    ref = fb.DeviceLayer(layer, max_batch=2)
    x = dev(I.workload_x(2, layer, 2))
    y_ref = torch.empty((2, layer.n), dtype=torch.int16, device="cuda")
    ref.gemv(x, y_ref)
    d = ref.make_desc()
    d.workspace, d.workspace_bytes = None, 0
    h = fb.fluxbin_create(d)
    y = torch.zeros_like(y_ref)
    st = fb.raw_status("fluxbin_gemv", ctypes.c_void_p(h), ctypes.c_void_p(x.data_ptr()),
                       ctypes.c_void_p(y.data_ptr()), ctypes.c_int64(2), None)
    assert st == fb.ERR_WORKSPACE
    fb.fluxbin_gemv_static(h, x, y, 2)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
    fb.fluxbin_destroy(h)
    ref.close()


def test_static_scratch_under_graph_capture(fb):
    note("static scratch: captured in a graph, 3 replays with eager work between")
    layer = I.workload_layer(2)
    dl = fb.DeviceLayer(layer)
    xs = [dev(I.workload_x(2, layer, 1, layer=i)) for i in range(2)]
    eager = []
    for x in xs:
        y = torch.empty((1, layer.n), dtype=torch.int16, device="cuda")
        dl.gemv(x, y)
        eager.append(y)
    torch.cuda.synchronize()
    outs = [torch.zeros((1, layer.n), dtype=torch.int16, device="cuda") for _ in xs]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for x, o in zip(xs, outs):
                fb.fluxbin_gemv_static(dl.handle, x, o, 1, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        for o in outs:
            o.zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), f"replay {rep}"
        del junk
    dl.close()


def test_static_scratch_size_limit(fb):
    note("static scratch: beyond 2^20 words is rejected, within runs")
    layer = I.make_layer(131072, 256, 2, 0, 4, seed=(78, 0, 0))
    dl = fb.DeviceLayer(layer, max_batch=9, chunks_per_block=1)
    assert dl.plan["splits"] > 1
    x = dev(I.make_x(layer, 9, seed=(78, 0, 0)))
    y = torch.zeros((9, layer.n), dtype=torch.int16, device="cuda")
    with pytest.raises(fb.FluxbinError) as ei:
        fb.fluxbin_gemv_static(dl.handle, x, y, 9)  # 9 x 131072 words > 2^20
    assert ei.value.status == fb.ERR_UNSUPPORTED and "static scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert int(y.abs().sum()) == 0  # nothing launched
    y0, y1 = both(fb, dl, x[:8], 8)  # 8 x 131072 = 2^20 words: the limit itself
    assert torch.equal(y0, y1)
    dl.close()
