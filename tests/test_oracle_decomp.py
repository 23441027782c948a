"""Pins of the oracle's offline decomposition W ~ sum_b diag(r_b) B_b diag(c_b).

The pages fix what each step minimises (FluxBin summary, section 3 "Parameter Optimization";
appendix A.1: with B and the column scales fixed each row scale is a scalar least-squares
problem with a closed form, and symmetrically for the columns; appendix A.2: with the scales
fixed, an exhaustive search over the Kb signs of each element is globally optimal).  Each
test checks that property with numpy, independently of the oracle's arithmetic: the error is a
quadratic in one scale whose vertex must sit at the step's value; brute-force enumeration of
every sign combination; a never-increasing error over the steps; exact recovery of a matrix
that is exactly one scaled binary basis; the pages' standard binarisation scale (mean |W|)
for the first basis.
"""
import itertools

import numpy as np
import pytest

from binary_basis_lut_amd import inputs as I

from .test_oracle_pins import bits_of


def signs_of(bits, k):
    """canonical words [kb][n][w] -> +-1 float [kb][n][k] (numpy bit unpacking)."""
    return np.stack([2.0 * bits_of(b, k) - 1.0 for b in bits])


def w_hat(bits, r, c, k, skip=None):
    s = signs_of(bits, k)
    out = np.zeros(s.shape[1:])
    for b in range(s.shape[0]):
        if b != skip:
            out += r[b][:, None] * s[b] * c[b][None, :]
    return out


def wf(w):
    return np.asarray(w).view(np.float16).astype(np.float64)


def err(w, bits, r, c, d=None):
    k = w.shape[1]
    res = wf(w) - w_hat(bits, r, c, k)
    return float(((res * res) * (1.0 if d is None else d[None, :])).sum())


def random_state(n, k, kb, seed):
    rng = I.stream(80, n, k, kb, seed)
    w = I.decomp_matrix(n, k, seed=(80, n, k))
    bits = np.stack([I.sign_words(rng, n, k) for _ in range(kb)])
    r = np.abs(rng.normal(0.02, 0.01, (kb, n))) + 1e-3
    c = np.abs(rng.normal(1.0, 0.3, (kb, k))) + 0.05
    return w, bits, r, c


def vertex_offset(f, x0, h):
    """Position of the vertex of the quadratic through f(x0 - h), f(x0), f(x0 + h), relative to x0, in units of h."""
    fm, f0, fp = f(x0 - h), f(x0), f(x0 + h)
    curv = fp + fm - 2 * f0
    assert curv > 0
    return (fm - fp) / (2 * curv)


@pytest.mark.parametrize("kb,basis", [(1, 0), (2, 1), (3, 0), (4, 2)])
@pytest.mark.parametrize("weighted", [False, True])
def test_row_step_is_the_least_squares_vertex(orc, kb, basis, weighted):
    n, k = 9, 70
    w, bits, r, c = random_state(n, k, kb, basis)
    d = I.calibration_weights(k, 0.05, seed=(81, k)) if weighted else None
    rn = orc.decomp_row_scales(w, kb, basis, bits, r, c, d)
    for i in (0, 4, n - 1):
        def f(t):
            rr = r.copy()
            rr[basis] = rn
            rr[basis, i] = t
            return err(w, bits, rr, c, d)
        assert abs(vertex_offset(f, rn[i], 0.05)) < 1e-7


@pytest.mark.parametrize("kb,basis", [(1, 0), (2, 0), (3, 2), (4, 3)])
def test_column_step_is_the_least_squares_vertex(orc, kb, basis):
    n, k = 40, 37
    w, bits, r, c = random_state(n, k, kb, basis + 10)
    cn = orc.decomp_col_scales(w, kb, basis, bits, r, c)
    d = I.calibration_weights(k, 0.05, seed=(82, k))
    for j in (0, 20, k - 1):
        for dd in (None, d):  # the column weight cancels: the same vertex with or without it
            def f(t):
                cc = c.copy()
                cc[basis] = cn
                cc[basis, j] = t
                return err(w, bits, r, cc, dd)
            assert abs(vertex_offset(f, cn[j], 0.2)) < 1e-7


def dyadic_scales(rng, kb, n, k):
    r = rng.choice([0.25, 0.5, 1.0], size=(kb, n))
    c = rng.choice([0.125, 0.25, 0.5, 1.0], size=(kb, k))
    return r, c


@pytest.mark.parametrize("kb", [1, 2, 3, 4])
def test_sign_step_is_the_exhaustive_optimum_with_smallest_index_ties(orc, kb):
    """Dyadic values: every candidate error is exact, so ties are real; the chosen combination must be
    the smallest index among the exact minima (bit b of the index set = +1 on basis b)."""
    n, k = 6, 40
    rng = I.stream(83, kb)
    r, c = dyadic_scales(rng, kb, n, k)
    w = (rng.integers(-16, 17, size=(n, k)) * 0.0625).astype(np.float16).view(np.uint16)
    bits = orc.decomp_signs(w, kb, r, c)
    s = signs_of(bits, k)
    ties = 0
    for i in range(n):
        for j in range(k):
            errs = []
            for m in range(1 << kb):
                v = sum((1.0 if (m >> b) & 1 else -1.0) * r[b, i] * c[b, j] for b in range(kb))
                errs.append(abs(wf(w)[i, j] - v))
            best = min(errs)
            want = errs.index(best)
            ties += errs.count(best) > 1
            got = sum(1 << b for b in range(kb) if s[b, i, j] > 0)
            assert got == want, (i, j, errs)
    assert ties > 0  # the case exercises the tie rule


@pytest.mark.parametrize("kb", [2, 3])
def test_sign_step_on_random_scales_reaches_the_minimum(orc, kb):
    n, k = 8, 64
    w, bits, r, c = random_state(n, k, kb, 5)
    out = orc.decomp_signs(w, kb, r, c)
    chosen = np.abs(wf(w) - w_hat(out, r, c, k))
    combos = np.array(list(itertools.product([-1.0, 1.0], repeat=kb)))          # [2^kb][kb]
    p = r[:, :, None] * c[:, None, :]                                          # [kb][n][k]
    cand = np.abs(wf(w)[None] - np.einsum("mb,bij->mij", combos, p))
    assert np.all(chosen <= cand.min(axis=0) * (1 + 1e-14) + 1e-300)


@pytest.mark.parametrize("kb", [1, 2, 4])
def test_residual_signs(orc, kb):
    n, k = 7, 45
    w, bits, r, c = random_state(n, k, kb, 6)
    for basis in range(kb):
        got = orc.decomp_residual_signs(w, kb, basis, bits, r, c)
        res = wf(w) - w_hat(bits, r, c, k, skip=basis)
        assert np.array_equal(bits_of(got, k), (res >= 0).astype(np.int64))


def test_error_matches_numpy(orc):
    w, bits, r, c = random_state(12, 100, 3, 7)
    d = I.calibration_weights(100, 0.02, seed=(84, 0))
    assert np.isclose(orc.decomp_error(w, 3, bits, r, c), err(w, bits, r, c), rtol=1e-12)
    assert np.isclose(orc.decomp_error(w, 3, bits, r, c, d), err(w, bits, r, c, d), rtol=1e-12)


@pytest.mark.parametrize("n,k,kb,iters,weighted", [(33, 70, 1, 3, False), (64, 256, 2, 4, False),
                                                   (20, 129, 3, 3, True), (17, 64, 4, 2, True)])
def test_error_never_increases_over_the_steps(orc, n, k, kb, iters, weighted):
    w = I.decomp_matrix(n, k, seed=(85, n, k))
    d = I.calibration_weights(k, 0.02, seed=(85, k)) if weighted else None
    res = orc.decompose(w, kb, iters, d)
    t = res["trace"]
    assert t.size == 2 + iters * (2 * kb + 1)
    steps = np.diff(t[:-1])
    assert np.all(steps <= 1e-12 * t[0]), steps
    assert t[-2] < t[0]  # the iterations improve on the initialisation
    # the trace's last entry is the error of the returned (fp16-rounded) decomposition
    r16, c16 = wf(res["r16"]), wf(res["c16"])
    assert np.isclose(t[-1], err(w, res["bits"], r16, c16, d), rtol=1e-12)
    assert np.array_equal(res["r16"], res["r64"].astype(np.float16).view(np.uint16))
    assert np.array_equal(res["c16"], res["c64"].astype(np.float16).view(np.uint16))
    # the returned signs are the sign step against the rounded scales
    assert np.array_equal(res["bits"], orc.decomp_signs(w, kb, r16, c16))


def test_first_basis_starts_from_the_mean_absolute_value(orc):
    """Basis 0 after initialisation: B = sign(W), row scale = mean_j |W_ij| (the standard binarisation
    scale of the pages' related-work paragraph, per row), column scale = the column least squares."""
    n, k = 30, 50
    w = I.decomp_matrix(n, k, seed=(86, 0, 0))
    res = orc.decompose(w, 1, 0)
    a = np.abs(wf(w))
    r0 = a.mean(axis=1)
    assert np.allclose(res["r64"][0], r0, rtol=1e-14)
    assert np.allclose(res["c64"][0], (a * r0[:, None]).sum(axis=0) / (r0 * r0).sum(), rtol=1e-13)


def test_exact_single_basis_matrix_is_recovered(orc):
    """W = diag(u) S diag(v) with S = +-1: one basis represents it exactly."""
    n, k = 24, 96
    rng = I.stream(87)
    u = rng.choice([0.5, 1.0, 2.0], size=n) * 2.0 ** -6
    v = rng.choice([0.25, 0.5, 1.0], size=k)
    s = rng.choice([-1.0, 1.0], size=(n, k))
    w = (u[:, None] * s * v[None, :]).astype(np.float16).view(np.uint16)
    assert np.array_equal(wf(w), u[:, None] * s * v[None, :])
    res = orc.decompose(w, 1, 2)
    assert res["trace"][0] <= 1e-28 * (wf(w) ** 2).sum()
    assert np.array_equal(signs_of(res["bits"], k)[0], s)
    rec = w_hat(res["bits"], wf(res["r16"]), wf(res["c16"]), k)
    assert np.all(np.abs(rec - wf(w)) <= 2.0 ** -10 * np.abs(wf(w)))


def test_column_weights_uniform_scale_is_neutral_and_nonuniform_is_optimal(orc):
    n, k, kb = 16, 80, 2
    w, bits, r, c = random_state(n, k, kb, 8)
    d = I.calibration_weights(k, 0.05, seed=(88, k))
    r_none = orc.decomp_row_scales(w, kb, 1, bits, r, c)
    r_three = orc.decomp_row_scales(w, kb, 1, bits, r, c, np.full(k, 3.0))
    assert np.allclose(r_none, r_three, rtol=1e-14)
    r_d = orc.decomp_row_scales(w, kb, 1, bits, r, c, d)
    rr_d, rr_none = r.copy(), r.copy()
    rr_d[1], rr_none[1] = r_d, r_none
    assert err(w, bits, rr_d, c, d) <= err(w, bits, rr_none, c, d)
    assert not np.allclose(r_d, r_none, rtol=1e-6)
