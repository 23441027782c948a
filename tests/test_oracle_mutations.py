"""Plant plausible mistakes in copies of the oracle and check that the pins catch each one.

Each mutant is the oracle source with one textual change (a flipped sign
convention, a reversed bit order, a dropped term, a wrong index, a transposed
operand), compiled with gcc into a temporary directory.  The checks below are
the same closed forms, brute force and special cases as the pin tests, written
as predicates so that a mutant's failure can be observed instead of raised.
"""
import importlib.util
import os
import subprocess

import numpy as np
import pytest

from binary_basis_lut_amd import inputs as I

from . import test_oracle_decomp as D
from . import test_oracle_tables as T
from .test_oracle_grouped import exact_y_grouped
from .test_oracle_pins import bits_of, exact_y, f16, layer_from

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "fluxbin_oracle.c")
PY = os.path.join(ROOT, "oracle", "oracle.py")

MUTANTS = {
    "sign_convention_flipped": ("return ((w >> (col & 31)) & 1u) ? 1.0 : -1.0;",
                                "return ((w >> (col & 31)) & 1u) ? -1.0 : 1.0;"),
    "msb_first_bit_order": ("return ((w >> (col & 31)) & 1u) ? 1.0 : -1.0;",
                            "return ((w >> (31 - (col & 31))) & 1u) ? 1.0 : -1.0;"),
    "salient_term_dropped": ("wrow[L->idx[c]] += r * sign_at(row, c) * cs[(int64_t)b * L->s + c];",
                             "(void)row; (void)r;"),
    "salient_ungathered_column": ("wrow[L->idx[c]] += r * sign_at(row, c) * cs[(int64_t)b * L->s + c];",
                                  "wrow[c] += r * sign_at(row, c) * cs[(int64_t)b * L->s + c];"),
    "salient_scale_indexed_by_column": ("wrow[L->idx[c]] += r * sign_at(row, c) * cs[(int64_t)b * L->s + c];",
                                        "wrow[L->idx[c]] += r * sign_at(row, c) * cs[(int64_t)b * L->s + L->idx[c] % L->s];"),
    "last_basis_dropped": ("for (int32_t b = 0; b < L->kb; ++b) {", "for (int32_t b = 0; b + 1 < L->kb; ++b) {"),
    "row_scale_transposed": ("const uint16_t *rrow = L->r_g + ((int64_t)b * L->n + i) * L->ngroups;",
                             "const uint16_t *rrow = L->r_g + ((int64_t)b * L->n + (i * 7 + 1) % L->n) * L->ngroups;"),
    "column_scale_wrong_basis": ("wrow[j] += r * sign_at(row, j) * cg[(int64_t)b * L->k + j];",
                                 "wrow[j] += r * sign_at(row, j) * cg[j];"),
    "product_not_accumulated": ("acc += p;\n          am += fabs(p);", "acc = p;\n          am += fabs(p);"),
    "half_rounding_truncates": ("double q = rint(ldexp(a, 10 - e));", "double q = floor(ldexp(a, 10 - e));"),
    "grouped_salient_scale_by_compact_column": ("rrow[group_of(L->row_group, L->idx[c])]",
                                                "rrow[group_of(L->row_group, c)]"),
    "grouped_global_scale_first_group_only": ("double r = orc_half_to_double(rrow[group_of(L->row_group, j)]);",
                                              "double r = orc_half_to_double(rrow[0]);"),
    "grouped_scales_of_first_basis": ("const uint16_t *rrow = L->r_g + ((int64_t)b * L->n + i) * L->ngroups;",
                                      "const uint16_t *rrow = L->r_g + ((int64_t)0 * L->n + i) * L->ngroups;"),
    "grouped_group_boundary_off_by_one": ("{ return row_group ? j / row_group : 0; }",
                                          "{ return row_group ? (j > 0 ? (j - 1) / row_group : 0) : 0; }"),
    "decomp_row_denominator_not_squared": ("den += (d ? d[j] : 1.0) * cb[j] * cb[j];",
                                           "den += (d ? d[j] : 1.0) * cb[j];"),
    "decomp_row_residual_keeps_own_basis": (
        "approx_at(n, k, kb, bits, r, c, i, j, basis);\n      num += (d ? d[j] : 1.0)",
        "approx_at(n, k, kb, bits, r, c, i, j, -1);\n      num += (d ? d[j] : 1.0)"),
    "decomp_col_denominator_not_squared": ("den += rb[i] * rb[i];", "den += rb[i];"),
    "decomp_col_ignores_row_scale": ("num += res * sign_at(row, j) * rb[i];", "num += res * sign_at(row, j);"),
    "decomp_sign_ties_to_largest": ("if (e < best) {", "if (e <= best) {"),
    "decomp_sign_skips_last_basis": ("for (int32_t b = 0; b < kb; ++b) {\n          double p",
                                     "for (int32_t b = 0; b + 1 < kb; ++b) {\n          double p"),
    "decomp_weights_ignored": ("num += (d ? d[j] : 1.0) * res * sign_at(row, j) * cb[j];",
                               "num += res * sign_at(row, j) * cb[j];"),
    "table_fp16_rounding_skipped": ("double h = orc_half_to_double(orc_double_to_half((double)t));",
                                    "double h = (double)t;"),
    "table_summed_in_fp64": ("float t = (float)v[g - 1];", "double t = v[g - 1];"),
    "table_negated_half_misplaced": ("lut[(half - 1) ^ q] = -h;", "lut[q] = -h;"),
}


def build_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mpath = tmp_path / f"{name}.c"
    mpath.write_text(src.replace(old, new))
    so = tmp_path / f"lib_{name}.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-o", str(so),
                    str(mpath), "-lm"], check=True)
    spec = importlib.util.spec_from_file_location(f"oracle_{name}", PY)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    import ctypes
    mod._lib = ctypes.CDLL(str(so))
    mod._declare(mod._lib)
    return mod


# ----------------------------------------------------------------- predicates

def chk_popcount(O):
    n, k = 9, 77
    words = I.sign_words(I.stream(11, n, k), n, k)
    lay = layer_from(n, k, 1, 0, 0, words[None], f16(np.ones((1, n))), f16(np.ones((1, k))))
    y, _ = O.gemv_dense(lay, f16(np.ones((1, k))))
    pc = np.array([sum(bin(int(w)).count("1") for w in row) for row in words])
    return np.array_equal(y[0], 2.0 * pc - k)


def chk_one_hot(O):
    n, k, j = 17, 64, 45
    rng = I.stream(13, j)
    words = I.sign_words(rng, n, k)
    r = f16(rng.uniform(0.5, 2.0, (1, n)))
    c = np.zeros((1, k))
    c[0, j] = 1.0
    lay = layer_from(n, k, 1, 0, 0, words[None], r, f16(c))
    y, _ = O.gemv_dense(lay, f16(np.full((1, k), 3.0)))
    signs = 2 * bits_of(words, k)[:, j] - 1
    return np.array_equal(y[0], r[0].view(np.float16).astype(np.float64) * signs * 3.0)


def chk_bruteforce(O):
    for (n, k, kb, ks, s) in [(6, 40, 2, 1, 9), (4, 64, 3, 2, 17)]:
        lay = I.dyadic_layer(n, k, kb, ks, 4, s, seed=n * 100 + k)
        x = I.dyadic_x(k, 2, seed=k)
        if not np.array_equal(O.gemv_dense(lay, x)[0], exact_y(lay, x)):
            return False
    return True


def chk_half_numpy(O):
    v = np.random.default_rng(1).normal(0, 1, 5000)
    return np.array_equal(O.double_to_half(v), v.astype(np.float16).view(np.uint16))


def chk_grouped_one_hot(O):
    """Block-wise format: only group q of one basis scaled equals the per-row product on that group."""
    n, k = 20, 512
    lay = I.make_grouped_layer(n, k, 2, 2, 4, 128, 8, seed=(39, 0, 0))
    x = I.make_x(lay, 1, seed=(39, 0, 0))
    rv = I.scales(I.stream(40), (n,))
    for basis, q in [(("g", 1), 2), (("s", 0), 1), (("s", 1), 3)]:
        r_g = np.zeros((2, n, 4), np.uint16)
        r_s = np.zeros((2, n, 4), np.uint16)
        rr_g = np.zeros((2, n), np.uint16)
        rr_s = np.zeros((2, n), np.uint16)
        (r_g if basis[0] == "g" else r_s)[basis[1], :, q] = rv
        (rr_g if basis[0] == "g" else rr_s)[basis[1]] = rv
        xm = x.copy()
        xm[:, :q * 128] = 0
        xm[:, (q + 1) * 128:] = 0
        grp = I.Layer(n, k, lay.s, 2, 2, 4, lay.bits_g, r_g, lay.c_g, lay.bits_s, r_s, lay.c_s, lay.sal_idx,
                      lay.outliers, 128, 8)
        row = I.Layer(n, k, lay.s, 2, 2, 4, lay.bits_g, rr_g, lay.c_g, lay.bits_s, rr_s, lay.c_s, lay.sal_idx)
        if not np.array_equal(O.gemv_dense(grp, x)[0], O.gemv_dense(row, xm)[0]):
            return False
    return True


def chk_grouped_bruteforce(O):
    lay = I.dyadic_grouped_layer(4, 384, 2, 2, 4, 128, 8, seed=5)
    x = I.dyadic_x(384, 1, seed=6)
    return np.array_equal(O.gemv_dense(lay, x)[0], exact_y_grouped(lay, x))


def chk_decomp_steps(O):
    """Row and column steps at their least-squares vertex (weighted rows), the sign step at the exhaustive
    optimum with smallest-index ties, and a never-increasing error trace."""
    w, bits, r, c = D.random_state(9, 70, 3, 1)
    d = I.calibration_weights(70, 0.05, seed=(81, 70))
    rn = O.decomp_row_scales(w, 3, 1, bits, r, c, d)
    cn = O.decomp_col_scales(w, 3, 2, bits, r, c)
    for i in (0, 8):
        def f(t):
            rr = r.copy()
            rr[1] = rn
            rr[1, i] = t
            return D.err(w, bits, rr, c, d)
        if not abs(D.vertex_offset(f, rn[i], 0.05)) < 1e-7:
            return False
    for j in (0, 69):
        def g(t):
            cc = c.copy()
            cc[2] = cn
            cc[2, j] = t
            return D.err(w, bits, r, cc)
        if not abs(D.vertex_offset(g, cn[j], 0.2)) < 1e-7:
            return False
    rng = I.stream(83, 3)
    rd, cd = D.dyadic_scales(rng, 3, 6, 40)
    wd = (rng.integers(-16, 17, size=(6, 40)) * 0.0625).astype(np.float16).view(np.uint16)
    s = D.signs_of(O.decomp_signs(wd, 3, rd, cd), 40)
    for i in range(6):
        for j in range(40):
            errs = [abs(D.wf(wd)[i, j] - sum((1.0 if (m >> b) & 1 else -1.0) * rd[b, i] * cd[b, j]
                                             for b in range(3))) for m in range(8)]
            if sum(1 << b for b in range(3) if s[b, i, j] > 0) != errs.index(min(errs)):
                return False
    t = O.decompose(I.decomp_matrix(20, 129, seed=(85, 20, 129)), 3, 2, d=None)["trace"]
    return bool(np.all(np.diff(t[:-1]) <= 1e-12 * t[0]))


def chk_fp16_tables(O):
    """Quantised (fp16) tables equal numpy's float32 sums cast to float16, with the negated half in place."""
    rng = I.stream(100, 8)
    for g in (4, 8):
        for _ in range(20):
            c = np.abs(rng.normal(0, 0.02, g)) + 1e-3
            x = rng.normal(0, 1, g) * rng.choice([1.0, 20.0], g)
            v = c.astype(np.float16).astype(np.float64) * x.astype(np.float16).astype(np.float64)
            if not np.array_equal(O.quantised_table(g, v, 1), T.numpy_table(g, v)):
                return False
    v = T.crafted_double_rounding_case()
    return bool(np.array_equal(O.quantised_table(4, v, 1), T.numpy_table(4, v)))


CHECKS = [chk_popcount, chk_one_hot, chk_bruteforce, chk_half_numpy, chk_grouped_one_hot, chk_grouped_bruteforce,
          chk_decomp_steps, chk_fp16_tables]


def test_unmutated_oracle_passes_every_check(orc):
    assert all(chk(orc) for chk in CHECKS)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_every_planted_mistake_is_caught(name, tmp_path):
    O = build_mutant(name, tmp_path)
    failed = [chk.__name__ for chk in CHECKS if not chk(O)]
    assert failed, f"mutant {name} passed every pin"
