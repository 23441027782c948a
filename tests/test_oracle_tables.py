"""Pins of the oracle's quantised-table LUT route (fp16 table entries; LUT Tensor Core notes,
section 3.1.3: table entries stored in a lower, uniform precision).

The entries are built as the kernel builds them: the half-table sum in fp32 in a fixed order,
rounded to fp16 (nearest even), the other half negated.  That route is a diagnostic for the GPU
tests (it mirrors the kernel's entry arithmetic); the contract of the fp16-table format is the
bound against the exact product.  Pins: the entries against numpy's own float32 arithmetic and
float16 cast (which only restates the rounding rule); the symmetry LUT[~p] = -LUT[p]; exactness
when every entry is representable in fp16 (dyadic inputs: the quantised route equals the exact
product); and the quantisation bound against the exact product on random inputs, which is the
pin that ties the route to the mathematics.
"""
import numpy as np
import pytest

from binary_basis_lut_amd import inputs as I

from .test_oracle_grouped import exact_y_grouped
from .test_oracle_pins import exact_y


def numpy_table(g, v):
    half = 1 << (g - 1)
    v32 = v.astype(np.float32)
    out = np.empty(1 << g)
    for q in range(half):
        t = v32[g - 1]
        for i in range(g - 1):
            t = np.float32(t + v32[i]) if (q >> i) & 1 else np.float32(t - v32[i])
        h = np.float64(np.float16(t))
        out[q | half] = h
        out[(half - 1) ^ q] = -h
    return out


@pytest.mark.parametrize("g", [2, 4, 8])
def test_fp16_entries_match_numpy_float32_then_float16(orc, g):
    rng = I.stream(100, g)
    for _ in range(50):
        c = np.abs(rng.normal(0, 0.02, g)) + 1e-3
        x = rng.normal(0, 1, g) * rng.choice([1.0, 20.0], g)
        v = c.astype(np.float16).astype(np.float64) * x.astype(np.float16).astype(np.float64)
        got = orc.quantised_table(g, v, 1)
        assert np.array_equal(got, numpy_table(g, v))
        p = np.arange(1 << g)
        assert np.array_equal(got[p ^ ((1 << g) - 1)], -got[p])
        # format 0 is the exact table
        assert np.array_equal(orc.quantised_table(g, v, 0), orc.lut_explicit(g, v))


def crafted_double_rounding_case():
    """v = (2^-11, 2^-30, 0, 1): the exact entry for q = 3 is 1 + 2^-11 + 2^-30 (rounds up to 1 + 2^-10 in
    fp16), but summed in fp32 it is the fp16 midpoint 1 + 2^-11, which rounds to even (1.0).  Every v_t
    is a product of two fp16 values (2^-30 = 2^-15 * 2^-15)."""
    return np.array([2.0 ** -11, 2.0 ** -30, 0.0, 1.0])


def test_entries_are_rounded_from_the_fp32_sum(orc):
    v = crafted_double_rounding_case()
    t = orc.quantised_table(4, v, 1)
    assert t[3 | 8] == 1.0 and t[(8 - 1) ^ 3] == -1.0
    assert np.array_equal(t, numpy_table(4, v))


@pytest.mark.parametrize("g,n,k,kb,ks,s", [(4, 40, 200, 2, 1, 20), (8, 16, 256, 3, 2, 40), (4, 9, 33, 1, 0, 0)])
def test_dyadic_inputs_are_exact_with_fp16_tables(orc, g, n, k, kb, ks, s):
    lay = I.dyadic_layer(n, k, kb, ks, g, s, seed=n + k + 3)
    x = I.dyadic_x(k, 2, seed=k + 3)
    assert np.array_equal(orc.gemv_lut_fp16_tables(lay, x), exact_y(lay, x))


def test_dyadic_block_wise_exact_with_fp16_tables(orc):
    lay = I.dyadic_grouped_layer(8, 384, 2, 2, 4, 128, 8, seed=4)
    x = I.dyadic_x(384, 2, seed=5)
    assert np.array_equal(orc.gemv_lut_fp16_tables(lay, x), exact_y_grouped(lay, x))


def magnitude(lay, x):
    """M = sum over segments of |r_i| * sum_cols |c_j x_j| (per-row scales)."""
    xd = x.view(np.float16).astype(np.float64)
    m = np.zeros((x.shape[0], lay.n))
    for b in range(lay.kb):
        m += np.abs(xd) @ np.abs(lay.c_g[b].view(np.float16).astype(np.float64))[:, None] * \
            np.abs(lay.r_g[b].view(np.float16).astype(np.float64))[None, :]
    for b in range(lay.ks):
        m += np.abs(xd[:, lay.sal_idx]) @ np.abs(lay.c_s[b].view(np.float16).astype(np.float64))[:, None] * \
            np.abs(lay.r_s[b].view(np.float16).astype(np.float64))[None, :]
    return m


@pytest.mark.parametrize("g", [4, 8])
def test_quantisation_error_bound(orc, g):
    """|y_q - y| <= (2^-11 + g 2^-24) M: each entry carries at most its fp32 summation error and one
    fp16 rounding of its magnitude, which is at most the sub-vector's sum of |v|."""
    lay = I.make_layer(200, 1024, 2, 1, g, s=96, outlier_frac=0.01, seed=(101, g, 0))
    x = I.make_x(lay, 2, seed=(101, g, 0))
    y, _ = orc.gemv_dense(lay, x)
    yq = orc.gemv_lut_fp16_tables(lay, x)
    bound = (2.0 ** -11 + g * 2.0 ** -24) * magnitude(lay, x)
    assert np.all(np.abs(yq - y) <= bound)
    assert np.any(yq != y)  # the quantisation is visible
