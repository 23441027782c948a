"""Python front end of the fp64 CPU oracle (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's CPU
baseline may import this module.  It loads ``fluxbin_oracle.c`` compiled with
gcc (see :func:`build`); it imports nothing from the GPU package, and the GPU
package imports nothing from here.

All inputs are numpy arrays; fp16 quantities travel as raw uint16 bits.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

HERE = Path(__file__).resolve().parent
SRC = HERE / "fluxbin_oracle.c"
LIB = HERE / "_build" / "libfluxbin_oracle.so"

_lib = None


def build(force: bool = True) -> Path:
    """Compile the oracle with gcc (IEEE semantics: no fast-math, no FMA contraction)."""
    if LIB.exists() and not force:
        return LIB
    LIB.parent.mkdir(parents=True, exist_ok=True)
    tmp = LIB.with_suffix(".so.tmp")
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-fvisibility=hidden", "-Wall", "-o", str(tmp), str(SRC), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not LIB.exists() or LIB.stat().st_mtime < SRC.stat().st_mtime:
            build()
        _lib = ctypes.CDLL(str(LIB))
        _declare(_lib)
    return _lib


P = ctypes.c_void_p
I64 = ctypes.c_int64
I32 = ctypes.c_int32


def _declare(L):
    L.orc_half_to_double.restype = ctypes.c_double
    L.orc_half_to_double.argtypes = [ctypes.c_uint16]
    L.orc_double_to_half.restype = ctypes.c_uint16
    L.orc_double_to_half.argtypes = [ctypes.c_double]
    L.orc_half_array_to_double.argtypes = [P, I64, P]
    L.orc_double_array_to_half.argtypes = [P, I64, P]
    L.orc_pack_rowmajor.restype = I64
    L.orc_pack_rowmajor.argtypes = [P, I64, I64, I64, P]
    L.orc_unpack_rowmajor.argtypes = [P, I64, I64, P]
    L.orc_tiled_words.restype = I64
    L.orc_tiled_words.argtypes = [I64, I64]
    L.orc_tile_words.argtypes = [P, I64, I64, P]
    L.orc_vcm_gather_bits.argtypes = [P, I64, I64, P, I64, P]
    L.orc_gemv_dense.restype = ctypes.c_int
    L.orc_gemv_dense.argtypes = [I64, I64, I64, I32, I32, I64, P, P, P, P, P, P, P, P, I64, P, I64, P, P, I32]
    L.orc_gemv_lut.restype = ctypes.c_int
    L.orc_gemv_lut.argtypes = [I64, I64, I64, I32, I32, I64, I32, P, P, P, P, P, P, P, P, I64, P, I64, P]
    L.orc_gemv_lut_tables.restype = ctypes.c_int
    L.orc_gemv_lut_tables.argtypes = [I64, I64, I64, I32, I32, I64, I32, I32, P, P, P, P, P, P, P, P, I64, P, I64, P]
    L.orc_quantised_table.argtypes = [I32, P, I32, P]
    L.orc_tiled_scale_elems.restype = I64
    L.orc_tiled_scale_elems.argtypes = [I64, I64, I64]
    L.orc_tile_scales.argtypes = [P, I64, I64, I64, P]
    L.orc_lut_explicit.argtypes = [I32, P, P]
    L.orc_half_luts.restype = ctypes.c_int
    L.orc_half_luts.argtypes = [I64, I64, I32, I32, I32, P, P, P, P, I64, P, P]
    L.orc_dense_f16_gemv.argtypes = [P, I64, I64, P, I64, P, P]
    L.orc_max_threads.restype = ctypes.c_int
    L.orc_decomp_row_scales.argtypes = [P, I64, I64, I32, I32, P, P, P, P, P]
    L.orc_decomp_col_scales.argtypes = [P, I64, I64, I32, I32, P, P, P, P]
    L.orc_decomp_signs.argtypes = [P, I64, I64, I32, P, P, P]
    L.orc_decomp_residual_signs.argtypes = [P, I64, I64, I32, I32, P, P, P, P]
    L.orc_decomp_error.restype = ctypes.c_double
    L.orc_decomp_error.argtypes = [P, I64, I64, I32, P, P, P, P]
    L.orc_decompose.restype = ctypes.c_int
    L.orc_decompose.argtypes = [P, I64, I64, I32, I32, P, P, P, P, P, P, P]


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- fp16

def half_to_double(h) -> np.ndarray:
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float64)
    lib().orc_half_array_to_double(_p(h), h.size, _p(out))
    return out


def double_to_half(v) -> np.ndarray:
    """Round-to-nearest-even fp64 -> fp16, returned as raw uint16 bits."""
    v = _c(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().orc_double_array_to_half(_p(v), v.size, _p(out))
    return out


# ---------------------------------------------------------------- bits

def pack_rowmajor(signs, cols: int | None = None):
    """int8 +-1 [rows][ld] -> (canonical words uint32 [rows][ceil(cols/32)], invalid count)."""
    signs = _c(signs, np.int8)
    rows, ld = signs.shape
    cols = ld if cols is None else cols
    out = np.empty((rows, (cols + 31) // 32), np.uint32)
    bad = lib().orc_pack_rowmajor(_p(signs), rows, cols, ld, _p(out))
    return out, int(bad)


def unpack_rowmajor(words, cols: int) -> np.ndarray:
    words = _c(words, np.uint32)
    rows = words.shape[0]
    out = np.empty((rows, cols), np.int8)
    lib().orc_unpack_rowmajor(_p(words), rows, cols, _p(out))
    return out


def tile_words(canon, cols: int) -> np.ndarray:
    """Canonical words [rows][ceil(cols/32)] -> tiled device layout (flat uint32)."""
    canon = _c(canon, np.uint32)
    rows = canon.shape[0]
    out = np.empty(lib().orc_tiled_words(rows, cols), np.uint32)
    lib().orc_tile_words(_p(canon), rows, cols, _p(out))
    return out


def tile_scales(canon, m: int) -> np.ndarray:
    """Row scales uint16 [rows][groups] -> tiled block-wise layout (flat uint16), m groups per chunk."""
    canon = _c(canon, np.uint16)
    rows, groups = canon.shape
    out = np.empty(lib().orc_tiled_scale_elems(rows, groups, m), np.uint16)
    lib().orc_tile_scales(_p(canon), rows, groups, m, _p(out))
    return out


def vcm_gather_bits(src, k: int, idx) -> np.ndarray:
    src = _c(src, np.uint32)
    idx = _c(idx, np.int32)
    rows = src.shape[0]
    s = idx.size
    out = np.empty((rows, (s + 31) // 32), np.uint32)
    lib().orc_vcm_gather_bits(_p(src), rows, k, _p(idx), s, _p(out))
    return out


def vcm_gather_values(src, idx) -> np.ndarray:
    """Value gather: dst[r][c] = src[r][idx[c]] (any dtype)."""
    return np.ascontiguousarray(np.asarray(src)[:, np.asarray(idx, dtype=np.int64)])


# ---------------------------------------------------------------- products

def _layer_arrays(layer):
    kb, ks = layer.kb, layer.ks
    bits_s = _c(layer.bits_s, np.uint32) if ks else np.zeros(1, np.uint32)
    r_s = _c(layer.r_s, np.uint16) if ks else np.zeros(1, np.uint16)
    c_s = _c(layer.c_s, np.uint16) if ks else np.zeros(1, np.uint16)
    idx = _c(layer.sal_idx, np.int32) if ks else np.zeros(1, np.int32)
    return (_c(layer.bits_g, np.uint32), _c(layer.r_g, np.uint16), _c(layer.c_g, np.uint16),
            bits_s, r_s, c_s, idx)


def _row_group(layer) -> int:
    return int(getattr(layer, "row_group", 0) or 0)


def gemv_dense(layer, x, rows=None, nthreads: int = 0):
    """fp64 y = W_hat x and mag = sum_j |W_hat_ij x_j|, each [batch][len(rows) or n].

    Row scales are per row ([basis][n]) or, when ``layer.row_group`` > 0,
    block-wise ([basis][n][ceil(k / row_group)]).
    """
    x = _c(x, np.uint16)
    batch = x.shape[0]
    arrs = _layer_arrays(layer)
    rows_a = None if rows is None else _c(rows, np.int64)
    nrows = layer.n if rows is None else rows_a.size
    y = np.empty((batch, nrows), np.float64)
    mag = np.empty((batch, nrows), np.float64)
    err = lib().orc_gemv_dense(layer.n, layer.k, layer.s, layer.kb, layer.ks, _row_group(layer),
                               *[_p(a) for a in arrs], _p(x), batch, _p(rows_a), nrows, _p(y), _p(mag), nthreads)
    if err:
        raise ValueError("row index out of range" if err == 1 else "negative row_group")
    return y, mag


def gemv_lut(layer, x, g: int | None = None, rows=None):
    """fp64 y via explicit 2^g-entry tables (the method's steps, no fused kernels)."""
    x = _c(x, np.uint16)
    batch = x.shape[0]
    arrs = _layer_arrays(layer)
    rows_a = None if rows is None else _c(rows, np.int64)
    nrows = layer.n if rows is None else rows_a.size
    y = np.empty((batch, nrows), np.float64)
    g = layer.g if g is None else g
    err = lib().orc_gemv_lut(layer.n, layer.k, layer.s, layer.kb, layer.ks, _row_group(layer), g,
                             *[_p(a) for a in arrs], _p(x), batch, _p(rows_a), nrows, _p(y))
    if err:
        raise ValueError("unsupported g" if err == 1 else "a sub-vector spans two row-scale groups")
    return y


def gemv_lut_fp16_tables(layer, x, rows=None):
    """fp64 LUT route with fp16 table entries built in fp32 as the kernel builds them (quantised tables)."""
    x = _c(x, np.uint16)
    batch = x.shape[0]
    arrs = _layer_arrays(layer)
    rows_a = None if rows is None else _c(rows, np.int64)
    nrows = layer.n if rows is None else rows_a.size
    y = np.empty((batch, nrows), np.float64)
    err = lib().orc_gemv_lut_tables(layer.n, layer.k, layer.s, layer.kb, layer.ks, _row_group(layer), layer.g, 1,
                                    *[_p(a) for a in arrs], _p(x), batch, _p(rows_a), nrows, _p(y))
    if err:
        raise ValueError("unsupported g or a sub-vector spans two row-scale groups")
    return y


def quantised_table(g: int, v, table_fmt: int = 1) -> np.ndarray:
    v = _c(v, np.float64)
    out = np.empty(1 << g, np.float64)
    lib().orc_quantised_table(g, _p(v), table_fmt, _p(out))
    return out


def lut_explicit(g: int, v) -> np.ndarray:
    v = _c(v, np.float64)
    out = np.empty(1 << g, np.float64)
    lib().orc_lut_explicit(g, _p(v), _p(out))
    return out


def half_luts(layer, x):
    """fp64 half tables [batch][sum_seg ceil(L/g) * 2^(g-1)] and the per-sub-vector sum |v|."""
    x = _c(x, np.uint16)
    batch = x.shape[0]
    g = layer.g
    nsub = layer.kb * ((layer.k + g - 1) // g) + layer.ks * ((layer.s + g - 1) // g)
    out = np.empty((batch, nsub * (1 << (g - 1))), np.float64)
    absv = np.empty((batch, nsub), np.float64)
    arrs = _layer_arrays(layer)
    err = lib().orc_half_luts(layer.k, layer.s, layer.kb, layer.ks, g, _p(arrs[2]), _p(arrs[5]),
                              _p(arrs[6]), _p(x), batch, _p(out), _p(absv))
    if err:
        raise ValueError("unsupported g")
    return out, absv


def dense_f16_gemv(w, x):
    w = _c(w, np.uint16)
    x = _c(x, np.uint16)
    n, k = w.shape
    batch = x.shape[0]
    y = np.empty((batch, n), np.float64)
    mag = np.empty((batch, n), np.float64)
    lib().orc_dense_f16_gemv(_p(w), n, k, _p(x), batch, _p(y), _p(mag))
    return y, mag


def max_threads() -> int:
    return int(lib().orc_max_threads())


# ---------------------------------------------------------------- tolerance

def contract_bound(mag) -> np.ndarray:
    """Per-row tolerance of the output: 1e-3 * sum_j |W_hat_ij x_j|."""
    return 1e-3 * np.asarray(mag)


def tight_bound(y_ref, mag) -> np.ndarray:
    """Diagnostic bound: fp16 output rounding plus fp32 accumulation, 2^-11 |y| + 2^-20 sum|W x|."""
    return np.abs(y_ref) * 2.0 ** -11 + np.asarray(mag) * 2.0 ** -20


# ---------------------------------------------------------------- offline decomposition
# W fp16 [n][k] (uint16 bits); bits canonical [kb][n][ceil(k/32)]; r fp64 [kb][n]; c fp64 [kb][k];
# d fp64 [k] column weights or None (all 1).

def _opt(a, dtype):
    return None if a is None else _c(a, dtype)


def decomp_row_scales(w, kb, basis, bits, r, c, d=None) -> np.ndarray:
    w = _c(w, np.uint16)
    n, k = w.shape
    out = np.empty(n, np.float64)
    bits, r, c, d = _c(bits, np.uint32), _c(r, np.float64), _c(c, np.float64), _opt(d, np.float64)
    lib().orc_decomp_row_scales(_p(w), n, k, kb, basis, _p(bits), _p(r), _p(c), _p(d), _p(out))
    return out


def decomp_col_scales(w, kb, basis, bits, r, c) -> np.ndarray:
    w = _c(w, np.uint16)
    n, k = w.shape
    out = np.empty(k, np.float64)
    bits, r, c = _c(bits, np.uint32), _c(r, np.float64), _c(c, np.float64)
    lib().orc_decomp_col_scales(_p(w), n, k, kb, basis, _p(bits), _p(r), _p(c), _p(out))
    return out


def decomp_signs(w, kb, r, c) -> np.ndarray:
    w = _c(w, np.uint16)
    n, k = w.shape
    out = np.empty((kb, n, (k + 31) // 32), np.uint32)
    r, c = _c(r, np.float64), _c(c, np.float64)
    lib().orc_decomp_signs(_p(w), n, k, kb, _p(r), _p(c), _p(out))
    return out


def decomp_residual_signs(w, kb, basis, bits, r, c) -> np.ndarray:
    w = _c(w, np.uint16)
    n, k = w.shape
    out = np.empty((n, (k + 31) // 32), np.uint32)
    bits, r, c = _c(bits, np.uint32), _c(r, np.float64), _c(c, np.float64)
    lib().orc_decomp_residual_signs(_p(w), n, k, kb, basis, _p(bits), _p(r), _p(c), _p(out))
    return out


def decomp_error(w, kb, bits, r, c, d=None) -> float:
    w = _c(w, np.uint16)
    n, k = w.shape
    bits, r, c, d = _c(bits, np.uint32), _c(r, np.float64), _c(c, np.float64), _opt(d, np.float64)
    return float(lib().orc_decomp_error(_p(w), n, k, kb, _p(bits), _p(r), _p(c), _p(d)))


def decompose(w, kb: int, iters: int, d=None) -> dict:
    """The whole decomposition: bits, fp16 r/c, the fp64 scales before rounding, the error trace."""
    w = _c(w, np.uint16)
    n, k = w.shape
    d = _opt(d, np.float64)
    bits = np.empty((kb, n, (k + 31) // 32), np.uint32)
    r16 = np.empty((kb, n), np.uint16)
    c16 = np.empty((kb, k), np.uint16)
    r64 = np.empty((kb, n), np.float64)
    c64 = np.empty((kb, k), np.float64)
    trace = np.empty(2 + iters * (2 * kb + 1), np.float64)
    err = lib().orc_decompose(_p(w), n, k, kb, iters, _p(d), _p(bits), _p(r16), _p(c16), _p(r64), _p(c64),
                              _p(trace))
    if err:
        raise ValueError("unsupported decomposition arguments")
    return {"bits": bits, "r16": r16, "c16": c16, "r64": r64, "c64": c64, "trace": trace}
