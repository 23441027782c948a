"""Pins of the fp64 oracle against what the pages and plain mathematics fix.

None of these tests compares the oracle with itself: each checks a closed
form, an exact integer brute force, an independent library routine (numpy's
float16 cast and bit unpacking), a special case that reduces to a simpler
problem, or the separately written LUT route.
"""
import json
import os

import numpy as np
import pytest

from binary_basis_lut_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bits_of(words: np.ndarray, cols: int) -> np.ndarray:
    """Canonical words -> 0/1 matrix via numpy's little-endian bit unpacking."""
    w = np.ascontiguousarray(words, dtype="<u4")
    b = np.unpackbits(w.view(np.uint8).reshape(w.shape[0], -1), axis=1, bitorder="little")
    return b[:, :cols].astype(np.int64)


def layer_from(n, k, kb, ks, s, bits_g, r_g, c_g, bits_s=None, r_s=None, c_s=None, idx=None, g=4):
    if not ks:
        bits_s = np.zeros((0, n, 0), np.uint32)
        r_s = np.zeros((0, n), np.uint16)
        c_s = np.zeros((0, 0), np.uint16)
        idx = np.zeros(0, np.int32)
        s = 0
    return I.Layer(n, k, s, kb, ks, g, np.asarray(bits_g, np.uint32), np.asarray(r_g, np.uint16),
                   np.asarray(c_g, np.uint16), np.asarray(bits_s, np.uint32), np.asarray(r_s, np.uint16),
                   np.asarray(c_s, np.uint16), np.asarray(idx, np.int32))


def f16(v):
    return np.asarray(v, np.float64).astype(np.float16).view(np.uint16)


# --------------------------------------------------------------------------- fp16

def test_half_to_double_all_patterns_match_numpy(orc):
    h = np.arange(1 << 16, dtype=np.uint16)
    mine = orc.half_to_double(h)
    ref = h.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert np.array_equal(np.signbit(mine[~nan]), np.signbit(ref[~nan]))


def test_double_to_half_rne_matches_numpy(orc):
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.normal(0, 1, 20000),
        rng.normal(0, 1e-5, 5000),                      # subnormal range
        rng.uniform(-70000, 70000, 5000),               # overflow range
        # exact ties: odd multiples of half a quantum at several binades
        (np.arange(1, 4001, 2) * 2.0 ** -11) * 0.5,
        (np.arange(1, 4001, 2) * 2.0 ** -24) * 0.5,
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, -65520.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26,
                  2.0 ** -14, 2.0 ** -14 * (1 - 2.0 ** -12), np.inf, -np.inf]),
    ])
    mine = orc.double_to_half(v)
    ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(mine, ref)


# --------------------------------------------------------------------------- closed forms

@pytest.mark.parametrize("n,k", [(5, 77), (33, 32), (64, 128), (7, 1)])
def test_popcount_identity(orc, n, k):
    """K_b = 1, r = c = 1, x = 1: y_i = 2 * popcount(row_i) - K exactly (pins sign convention and padding)."""
    rng = I.stream(11, n, k)
    words = I.sign_words(rng, n, k)
    lay = layer_from(n, k, 1, 0, 0, words[None], f16(np.ones((1, n))), f16(np.ones((1, k))))
    x = f16(np.ones((1, k)))
    y, mag = orc.gemv_dense(lay, x)
    pc = np.array([sum(bin(int(w)).count("1") for w in row) for row in words])
    assert np.array_equal(y[0], 2.0 * pc - k)
    assert np.array_equal(mag[0], np.full(n, float(k)))


def test_two_bases_popcount(orc):
    """Second basis with r = 1/2: y = (2 pc0 - K) + (2 pc1 - K) / 2 exactly."""
    n, k = 9, 100
    rng = I.stream(12)
    w0, w1 = I.sign_words(rng, n, k), I.sign_words(rng, n, k)
    r = f16(np.stack([np.ones(n), np.full(n, 0.5)]))
    lay = layer_from(n, k, 2, 0, 0, np.stack([w0, w1]), r, f16(np.ones((2, k))))
    y, _ = orc.gemv_dense(lay, f16(np.ones((1, k))))
    pc = lambda W: np.array([sum(bin(int(w)).count("1") for w in row) for row in W])
    assert np.array_equal(y[0], (2.0 * pc(w0) - k) + 0.5 * (2.0 * pc(w1) - k))


@pytest.mark.parametrize("j", [0, 1, 31, 32, 45, 63])
def test_one_hot_column_selects_sign(orc, j):
    """c = e_j: y_i = r_i * sign(B_ij) * x_j, which fixes column and bit order."""
    n, k = 17, 64
    rng = I.stream(13, j)
    words = I.sign_words(rng, n, k)
    r = f16(rng.uniform(0.5, 2.0, (1, n)))
    c = np.zeros((1, k))
    c[0, j] = 1.0
    lay = layer_from(n, k, 1, 0, 0, words[None], r, f16(c))
    x = f16(np.full((1, k), 3.0))
    y, _ = orc.gemv_dense(lay, x)
    signs = 2 * bits_of(words, k)[:, j] - 1
    assert np.array_equal(y[0], orc.half_to_double(r[0]) * signs * 3.0)


def test_fig3_worked_shape(orc):
    """LUT Tensor Core notes, section 2.2 Figure 3: 1x4 activations, a 4xN 1-bit block, one 16-entry table."""
    fx = json.load(open(os.path.join(GOLDEN, "fig3_lut_1x4.json")))
    table = np.array(fx["table"], np.float64)
    # the explicit table for x = (1, 2, 4, 8)
    assert np.array_equal(orc.lut_explicit(4, np.array(fx["x"])), table)
    # N = 16 weight columns (rows of B here), column p carries pattern p; r = c = 1
    n, k = 16, 4
    words = np.arange(16, dtype=np.uint32)[:, None]
    lay = layer_from(n, k, 1, 0, 0, words[None], f16(np.ones((1, n))), f16(np.ones((1, k))))
    x = f16(np.array([fx["x"]]))
    y, _ = orc.gemv_dense(lay, x)
    assert np.array_equal(y[0], table)
    assert np.array_equal(orc.gemv_lut(lay, x, g=4)[0], table)


@pytest.mark.parametrize("g", [1, 2, 4, 8])
def test_half_table_closed_form(orc, g):
    """With v_t = 2^t the stored half entry q (pattern q | 2^(g-1)) equals 2q + 1."""
    k = g
    lay = layer_from(1, k, 1, 0, 0, np.zeros((1, 1, 1), np.uint32), f16([[1.0]]), f16(np.ones((1, k))), g=g)
    x = f16(np.array([[2.0 ** t for t in range(g)]]))
    half, absv = orc.half_luts(lay, x)
    assert np.array_equal(half[0], 2.0 * np.arange(1 << (g - 1)) + 1.0)
    assert absv[0, 0] == (1 << g) - 1


@pytest.mark.parametrize("g", [2, 4, 8])
def test_lut_symmetry_bit_exact(orc, g):
    """LUT[~p] == -LUT[p] exactly (LUT Tensor Core notes, section 3.1.2)."""
    rng = np.random.default_rng(g)
    for _ in range(20):
        v = rng.normal(0, 1, g) * rng.choice([1e-3, 1.0, 1e3], g)
        lut = orc.lut_explicit(g, v)
        p = np.arange(1 << g)
        assert np.array_equal(lut[(~p) & ((1 << g) - 1)], -lut[p])


# --------------------------------------------------------------------------- brute force

def exact_y(layer, x):
    """Exact rational y for dyadic inputs, with Python integers (scaled by 2^12)."""
    n, k = layer.n, layer.k
    xs = (np.asarray(x).view(np.float16).astype(np.float64) * 8).astype(np.int64)       # x * 2^3
    out = []
    for b in range(xs.shape[0]):
        row_vals = []
        for i in range(n):
            tot = 0
            for kb in range(layer.kb):
                bits = bits_of(layer.bits_g[kb][i:i + 1], k)[0]
                r = int(layer.r_g[kb][i:i + 1].view(np.float16)[0] * 2)             # r * 2
                c = (layer.c_g[kb].view(np.float16).astype(np.float64) * 4).astype(np.int64)  # c * 4
                tot += r * sum(int(2 * bits[j] - 1) * int(c[j]) * int(xs[b, j]) for j in range(k))
            for sb in range(layer.ks):
                bits = bits_of(layer.bits_s[sb][i:i + 1], layer.s)[0]
                r = int(layer.r_s[sb][i:i + 1].view(np.float16)[0] * 2)
                c = (layer.c_s[sb].view(np.float16).astype(np.float64) * 4).astype(np.int64)
                tot += r * sum(int(2 * bits[cc] - 1) * int(c[cc]) * int(xs[b, layer.sal_idx[cc]])
                               for cc in range(layer.s))
            row_vals.append(tot / 64.0)   # undo 2 * 4 * 8
        out.append(row_vals)
    return np.array(out)


@pytest.mark.parametrize("n,k,kb,ks,s", [(6, 40, 2, 1, 9), (4, 64, 3, 2, 17), (3, 33, 1, 1, 33), (5, 20, 2, 0, 0)])
def test_integer_bruteforce_dyadic(orc, n, k, kb, ks, s):
    lay = I.dyadic_layer(n, k, kb, ks, 4, s, seed=n * 100 + k)
    x = I.dyadic_x(k, 2, seed=k)
    y, _ = orc.gemv_dense(lay, x)
    assert np.array_equal(y, exact_y(lay, x))
    assert np.array_equal(orc.gemv_lut(lay, x), exact_y(lay, x))


@pytest.mark.parametrize("g", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("seed", range(4))
def test_lut_route_matches_dense(orc, g, seed):
    rng = I.stream(21, g, seed)
    n = int(rng.integers(1, 40))
    k = int(rng.integers(1, 70))
    kb = int(rng.integers(1, 5))
    ks = int(rng.integers(0, 3))
    s = int(rng.integers(1, k + 1)) if ks else 0
    lay = I.make_layer(n, k, kb, ks, g, s=s if ks else None, seed=(21, g, seed))
    x = I.make_x(lay, 3, seed=(21, g, seed))
    yd, mag = orc.gemv_dense(lay, x)
    yl = orc.gemv_lut(lay, x, g=g)
    assert np.all(np.abs(yd - yl) <= 1e-12 * mag + 1e-300)


# --------------------------------------------------------------------------- VCM special cases

def test_vcm_all_columns_equals_extra_global_basis(orc):
    """S = every column: the salient basis is exactly one more global basis."""
    n, k = 20, 96
    rng = I.stream(31)
    wg = np.stack([I.sign_words(rng, n, k) for _ in range(2)])
    ws = I.sign_words(rng, n, k)[None]
    rg, cg = I.scales(rng, (2, n)), I.scales(rng, (2, k))
    rs, cs = I.scales(rng, (1, n)), I.scales(rng, (1, k))
    idx = np.arange(k, dtype=np.int32)
    hyb = layer_from(n, k, 2, 1, k, wg, rg, cg, ws, rs, cs, idx)
    glob = layer_from(n, k, 3, 0, 0, np.concatenate([wg, ws]), np.concatenate([rg, rs]), np.concatenate([cg, cs]))
    x = I.activations(rng, 2, k, np.zeros(0, np.int64))
    assert np.array_equal(orc.gemv_dense(hyb, x)[0], orc.gemv_dense(glob, x)[0])


def test_vcm_empty_is_global_only(orc):
    lay = I.make_layer(30, 64, 2, 1, 4, s=32, seed=(32, 0, 0))
    x = I.make_x(lay, 1, seed=(32, 0, 0))
    glob = layer_from(lay.n, lay.k, 2, 0, 0, lay.bits_g, lay.r_g, lay.c_g)
    zero_sal = layer_from(lay.n, lay.k, 2, 1, lay.s, lay.bits_g, lay.r_g, lay.c_g, lay.bits_s, lay.r_s,
                          np.zeros_like(lay.c_s), lay.sal_idx)
    assert np.array_equal(orc.gemv_dense(zero_sal, x)[0], orc.gemv_dense(glob, x)[0])


def test_vcm_compact_order_is_a_relabelling(orc):
    """Listing S in another order, with the compact bits and c_s permuted the same way, gives the same y."""
    n, k, s = 25, 80, 24
    lay = I.make_layer(n, k, 1, 1, 4, s=s, seed=(33, 0, 0))
    x = I.make_x(lay, 2, seed=(33, 0, 0))
    perm = I.stream(33, 1).permutation(s)
    signs = orc.unpack_rowmajor(lay.bits_s[0], s)[:, perm]
    bits_p, bad = orc.pack_rowmajor(signs)
    assert bad == 0
    lay_p = layer_from(n, k, 1, 1, s, lay.bits_g, lay.r_g, lay.c_g, bits_p[None], lay.r_s, lay.c_s[:, perm],
                       lay.sal_idx[perm])
    y0, mag = orc.gemv_dense(lay, x)
    y1, _ = orc.gemv_dense(lay_p, x)
    assert np.all(np.abs(y0 - y1) <= 1e-13 * mag)


def test_salient_reads_gathered_activations(orc):
    """Only x at the salient columns can change the salient term."""
    n, k, s = 12, 64, 8
    lay = I.make_layer(n, k, 1, 1, 4, s=s, seed=(34, 0, 0))
    lay_sal_only = layer_from(n, k, 1, 1, s, lay.bits_g, lay.r_g, np.zeros_like(lay.c_g), lay.bits_s, lay.r_s,
                              lay.c_s, lay.sal_idx)
    x = I.make_x(lay, 1, seed=(34, 0, 0))
    y0, _ = orc.gemv_dense(lay_sal_only, x)
    x2 = x.copy()
    others = np.setdiff1d(np.arange(k), lay.sal_idx)
    x2[0, others] = f16(np.full(others.size, 7.0))
    assert np.array_equal(orc.gemv_dense(lay_sal_only, x2)[0], y0)
    x3 = x.copy()
    x3[0, lay.sal_idx[3]] = f16([5.0])[0]
    assert not np.array_equal(orc.gemv_dense(lay_sal_only, x3)[0], y0)


# --------------------------------------------------------------------------- bits and layouts

@pytest.mark.parametrize("rows,cols", [(3, 1), (10, 31), (7, 32), (5, 33), (64, 200)])
def test_pack_roundtrip_and_invalid_count(orc, rows, cols):
    rng = np.random.default_rng(rows * cols)
    signs = rng.choice(np.array([-1, 1], np.int8), size=(rows, cols))
    words, bad = orc.pack_rowmajor(signs)
    assert bad == 0
    assert np.array_equal(orc.unpack_rowmajor(words, cols), signs)
    assert np.array_equal(2 * bits_of(words, cols) - 1, signs)
    # padding bits are zero
    if cols % 32:
        assert np.all(words[:, -1] >> np.uint32(cols % 32) == 0)
    bad_signs = signs.copy()
    bad_signs[0, 0] = 0
    bad_signs[-1, -1] = 5
    w2, bad2 = orc.pack_rowmajor(bad_signs)
    assert bad2 == 2 and (w2[0, 0] & 1) == 0


@pytest.mark.parametrize("rows,cols", [(1, 1), (64, 128), (65, 129), (130, 300), (200, 4096)])
def test_tiled_layout_matches_reshape_definition(orc, rows, cols):
    rng = I.stream(41, rows, cols)
    canon = I.sign_words(rng, rows, cols)
    rt, nc = -(-rows // 64), -(-cols // 128)
    pad = np.zeros((rt * 64, nc * 4), np.uint32)
    pad[:rows, :canon.shape[1]] = canon
    ref = pad.reshape(rt, 64, nc, 4).transpose(0, 2, 1, 3).reshape(-1)
    assert np.array_equal(orc.tile_words(canon, cols), ref)


@pytest.mark.parametrize("k,s", [(64, 10), (100, 32), (4096, 256), (33, 33)])
def test_vcm_gather_bits_matches_unpacked_gather(orc, k, s):
    rows = 9
    rng = I.stream(42, k, s)
    src = I.sign_words(rng, rows, k)
    idx = np.sort(rng.choice(k, s, replace=False)).astype(np.int32)
    dst = orc.vcm_gather_bits(src, k, idx)
    assert np.array_equal(bits_of(dst, s), bits_of(src, k)[:, idx])
    if s % 32:
        assert np.all(dst[:, -1] >> np.uint32(s % 32) == 0)


def test_batch_rows_are_independent(orc):
    lay = I.make_layer(40, 96, 2, 1, 4, s=32, seed=(43, 0, 0))
    x = I.make_x(lay, 5, seed=(43, 0, 0))
    y, _ = orc.gemv_dense(lay, x)
    for b in range(5):
        yb, _ = orc.gemv_dense(lay, x[b:b + 1])
        assert np.array_equal(yb[0], y[b])


def test_row_sampling_matches_full(orc):
    lay = I.make_layer(70, 64, 2, 1, 4, s=32, seed=(44, 0, 0))
    x = I.make_x(lay, 2, seed=(44, 0, 0))
    y, mag = orc.gemv_dense(lay, x)
    rows = np.array([69, 0, 5, 5, 33])
    ys, mags = orc.gemv_dense(lay, x, rows=rows)
    assert np.array_equal(ys, y[:, rows]) and np.array_equal(mags, mag[:, rows])
    with pytest.raises(ValueError):
        orc.gemv_dense(lay, x, rows=np.array([70]))


def test_dense_f16_reference(orc):
    """The dense fp16 context reference agrees with numpy's fp64 matmul of the same values."""
    rng = np.random.default_rng(5)
    w = rng.normal(0, 0.02, (33, 70)).astype(np.float16)
    x = rng.normal(0, 1, (2, 70)).astype(np.float16)
    y, mag = orc.dense_f16_gemv(w.view(np.uint16), x.view(np.uint16))
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.allclose(y, ref, rtol=0, atol=1e-12)
    assert np.allclose(mag, np.abs(x.astype(np.float64)[:, None, :] * w.astype(np.float64)[None]).sum(-1))
