"""GPU parity of the streamed workloads on every layer: the LLaMA-2-70B decode stream (80 layers x qkv,
o, gate+up, down; g = 4) and the LLaMA-2-7B stream (32 layers at g = 8), each layer drawn by the seeded
recipe (binary_basis_lut_amd.inputs) and uploaded one at a time.

Layer 0 of every shape is checked on all rows; every other layer on a deterministic 1/16 row sample
(rows congruent to the layer number modulo 16, so that the 16 residues are all visited), with the
contract and the rigorous rounding bound of test_gpu_parity.check_y against the fp64 oracle.
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


def stream_rows(n: int, layer_no: int):
    return None if layer_no == 0 else np.arange(layer_no % 16, n, 16)


def check_stream(fb, orc, wid: int, shape_idx: int):
    wl = I.WORKLOADS[wid]
    worst = (0.0, 0.0)
    for layer_no in range(wl.layers):
        note(f"workload {wid}: shape {wl.shapes[shape_idx].name} layer {layer_no}")
        layer = I.workload_layer(wid, shape_idx, layer_no)
        x = I.workload_x(wid, layer, 1, shape_idx, layer_no)
        dl = fb.DeviceLayer(layer)
        y16 = gemv(fb, dl, x)
        r = check_y(orc, layer, x, y16, dl.plan, rows=stream_rows(layer.n, layer_no))
        worst = (max(worst[0], r[0]), max(worst[1], r[1]))
        dl.close()
        del dl
    print(wl.shapes[shape_idx].name, f"{wl.layers} layers, worst ratios (contract, tight):", worst)


@pytest.mark.parametrize("shape_idx", [0, 1, 2, 3])
def test_llama70b_stream_every_layer(fb, orc, shape_idx):
    check_stream(fb, orc, 5, shape_idx)


@pytest.mark.parametrize("shape_idx", [0, 1, 2, 3])
def test_llama7b_g8_stream_every_layer(fb, orc, shape_idx):
    check_stream(fb, orc, 3, shape_idx)
