"""Seeded synthetic inputs shared by the GPU path's tests, the benchmark and the oracle's tests.

This module only draws numbers.  It holds none of the method's arithmetic: no
table building, no lookup, no scaling, no product.  Sign bases are drawn
directly as canonical packed words (uniform random bits, padding bits zero),
because drawing +-1 bytes first would need eight times the memory for the
70B-shaped layers.

Workload recipe (the synthetic stand-in for the FluxBin pages' LLaMA-2 7B/70B
layer shapes; no trained weights, datasets or calibration text are used):

* sign bits: uniform over {0, 1}, i.e. +-1 with probability 1/2 each;
* row and column scales: fp16(|N(0, 0.02)| + 1e-3), drawn in fp64, rounded to
  nearest-even by numpy's float16 cast;
* activations: fp16(N(0, 1)); optionally a set of outlier channels (1% of the
  input width, rounded) scaled by 20 before the cast;
* salient columns: 256 calibration draws of the same activation distribution,
  per-channel fp64 sample variance, the |S| largest (ties to the lower index),
  returned in ascending order.  This stands in for the pages' Hessian-guided
  search (which needs real calibration data); 256 is the pages' default
  calibration-set size (FluxBin summary, appendix D.4);
* |S| for a fraction f of K is f*K rounded up to a multiple of 32.

Block-wise row-scale layers (the pages' g128 storage, FluxBin summary,
appendix C.2) draw one row scale per (row, 128-column group) per basis from
the same distribution, and take their salient columns per group: the s
columns of largest calibration variance inside each group of 128 (ties to
the lower index), so that |S| = s * ceil(K / 128).

Every tensor has its own stream: numpy PCG64 seeded by
SeedSequence([base_seed, config, layer, linear, tensor]).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BASE_SEED = 0
NCAL = 256

# tensor ids inside one layer's seed tuple
T_BITS_G, T_R_G, T_C_G, T_BITS_S, T_R_S, T_C_S, T_X, T_OUTLIER, T_CAL = range(9)


def stream(*parts: int) -> np.random.Generator:
    """Independent PCG64 stream for the seed tuple (BASE_SEED, *parts)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([BASE_SEED, *parts])))


def words_per_row(cols: int) -> int:
    return (cols + 31) // 32


def sign_words(rng: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    """Uniform random canonical sign words uint32 [rows][ceil(cols/32)], padding bits zero."""
    w = words_per_row(cols)
    out = rng.integers(0, 1 << 32, size=(rows, w), dtype=np.uint64).astype(np.uint32)
    tail = cols % 32
    if tail and w:
        out[:, -1] &= np.uint32((1 << tail) - 1)
    return out


def scales(rng: np.random.Generator, shape) -> np.ndarray:
    """fp16(|N(0, 0.02)| + 1e-3) as raw uint16 bits."""
    v = np.abs(rng.normal(0.0, 0.02, size=shape)) + 1e-3
    return v.astype(np.float16).view(np.uint16)


def outlier_channels(rng: np.random.Generator, k: int, frac: float) -> np.ndarray:
    count = int(round(frac * k))
    if count == 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(rng.choice(k, size=count, replace=False)).astype(np.int64)


def activations(rng: np.random.Generator, batch: int, k: int, outliers: np.ndarray,
                mult: float = 20.0) -> np.ndarray:
    """fp16 [batch][k] as raw uint16 bits: N(0,1) with the outlier channels scaled."""
    v = rng.normal(0.0, 1.0, size=(batch, k))
    if outliers.size:
        v[:, outliers] *= mult
    return v.astype(np.float16).view(np.uint16)


def salient_count(k: int, frac: float) -> int:
    """frac*k rounded up to a multiple of 32 (0 stays 0)."""
    if frac <= 0:
        return 0
    return int(math.ceil(frac * k / 32.0)) * 32


def select_salient(rng: np.random.Generator, k: int, s: int, outliers: np.ndarray,
                   mult: float = 20.0) -> np.ndarray:
    """Top-|s| channels by fp64 sample variance of NCAL calibration draws, ascending int32."""
    if s == 0:
        return np.zeros(0, dtype=np.int32)
    cal = rng.normal(0.0, 1.0, size=(NCAL, k))
    if outliers.size:
        cal[:, outliers] *= mult
    cal = cal.astype(np.float16).astype(np.float64)
    var = cal.var(axis=0, ddof=1)
    order = np.lexsort((np.arange(k), -var))  # descending variance, ties to lower index
    return np.sort(order[:s]).astype(np.int32)


@dataclass
class Layer:
    """One linear layer's synthetic data (all host numpy arrays, fp16 as uint16 bits)."""
    n: int
    k: int
    s: int
    kb: int
    ks: int
    g: int
    bits_g: np.ndarray          # uint32 [kb][n][ceil(k/32)] canonical
    r_g: np.ndarray             # uint16 [kb][n]
    c_g: np.ndarray             # uint16 [kb][k]
    bits_s: np.ndarray          # uint32 [ks][n][ceil(s/32)] canonical
    r_s: np.ndarray             # uint16 [ks][n]
    c_s: np.ndarray             # uint16 [ks][s]
    sal_idx: np.ndarray         # int32 [s]
    outliers: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))
    # 0: one row scale per row per basis (r_g [kb][n], r_s [ks][n]).  Else the
    # block-wise format: r_g [kb][n][G], r_s [ks][n][G], G = ceil(k / row_group),
    # with sal_group salient columns taken from every group of row_group columns.
    row_group: int = 0
    sal_group: int = 0

    def packed_bytes(self) -> int:
        return (self.bits_g.nbytes + self.bits_s.nbytes)


def make_layer(n: int, k: int, kb: int, ks: int, g: int, sal_frac: float = 0.0,
               s: int | None = None, outlier_frac: float = 0.0,
               seed: tuple = (0, 0, 0)) -> Layer:
    """Draw one layer.  `seed` = (config, layer, linear)."""
    if s is None:
        s = salient_count(k, sal_frac) if ks else 0
    outl = outlier_channels(stream(*seed, T_OUTLIER), k, outlier_frac)
    bits_g = np.stack([sign_words(stream(*seed, T_BITS_G, b), n, k) for b in range(kb)]) if kb else \
        np.zeros((0, n, words_per_row(k)), np.uint32)
    r_g = scales(stream(*seed, T_R_G), (kb, n))
    c_g = scales(stream(*seed, T_C_G), (kb, k))
    if ks and s:
        sal = select_salient(stream(*seed, T_CAL), k, s, outl)
        bits_s = np.stack([sign_words(stream(*seed, T_BITS_S, b), n, s) for b in range(ks)])
        r_s = scales(stream(*seed, T_R_S), (ks, n))
        c_s = scales(stream(*seed, T_C_S), (ks, s))
    else:
        ks, s = 0, 0
        sal = np.zeros(0, np.int32)
        bits_s = np.zeros((0, n, 0), np.uint32)
        r_s = np.zeros((0, n), np.uint16)
        c_s = np.zeros((0, 0), np.uint16)
    return Layer(n, k, s, kb, ks, g, bits_g, r_g, c_g, bits_s, r_s, c_s, sal, outl)


def select_salient_grouped(rng: np.random.Generator, k: int, group: int, per_group: int, outliers: np.ndarray,
                           mult: float = 20.0) -> np.ndarray:
    """The per_group highest-variance channels of every `group`-column block, ascending int32."""
    cal = rng.normal(0.0, 1.0, size=(NCAL, k))
    if outliers.size:
        cal[:, outliers] *= mult
    var = cal.astype(np.float16).astype(np.float64).var(axis=0, ddof=1)
    picked = []
    for g0 in range(0, k, group):
        cols = np.arange(g0, min(g0 + group, k))
        if cols.size < per_group:
            raise ValueError(f"group at column {g0} has {cols.size} columns, fewer than {per_group}")
        order = np.lexsort((cols, -var[cols]))  # descending variance, ties to lower index
        picked.append(np.sort(cols[order[:per_group]]))
    return np.concatenate(picked).astype(np.int32)


def make_grouped_layer(n: int, k: int, kb: int, ks: int, g: int, row_group: int = 128, sal_group: int = 8,
                       outlier_frac: float = 0.0, seed: tuple = (0, 0, 0)) -> Layer:
    """Draw one layer in the block-wise row-scale format (`seed` = (config, layer, linear))."""
    ng = (k + row_group - 1) // row_group
    outl = outlier_channels(stream(*seed, T_OUTLIER), k, outlier_frac)
    bits_g = np.stack([sign_words(stream(*seed, T_BITS_G, b), n, k) for b in range(kb)])
    r_g = scales(stream(*seed, T_R_G), (kb, n, ng))
    c_g = scales(stream(*seed, T_C_G), (kb, k))
    if ks:
        sal = select_salient_grouped(stream(*seed, T_CAL), k, row_group, sal_group, outl)
        s = int(sal.size)
        bits_s = np.stack([sign_words(stream(*seed, T_BITS_S, b), n, s) for b in range(ks)])
        r_s = scales(stream(*seed, T_R_S), (ks, n, ng))
        c_s = scales(stream(*seed, T_C_S), (ks, s))
    else:
        s, sal_group = 0, 0
        sal = np.zeros(0, np.int32)
        bits_s = np.zeros((0, n, 0), np.uint32)
        r_s = np.zeros((0, n, ng), np.uint16)
        c_s = np.zeros((0, 0), np.uint16)
    return Layer(n, k, s, kb, ks, g, bits_g, r_g, c_g, bits_s, r_s, c_s, sal, outl, row_group, sal_group)


def make_x(layer: Layer, batch: int, seed: tuple = (0, 0, 0)) -> np.ndarray:
    """Activations for `layer` (same outlier channels as its calibration draws)."""
    return activations(stream(*seed, T_X, batch), batch, layer.k, layer.outliers)


# --------------------------------------------------------------------------
# The five workloads (LLaMA-2 7B / 70B layer shapes, synthetic data)
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class Shape:
    name: str
    k: int
    n: int


@dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    shapes: tuple
    kb: int
    ks: int
    g: int
    sal_frac: float
    sal_fixed: int | None
    outlier_frac: float
    layers: int
    batches: tuple


WORKLOADS = {
    1: Workload(1, "gemv_512x512_kb2_g4", (Shape("single", 512, 512),), 2, 0, 4, 0.0, None, 0.0, 1, (1,)),
    2: Workload(2, "llama2_7b_q_proj_4096x4096_kb2_ks1_s256_g4",
                (Shape("q_proj", 4096, 4096),), 2, 1, 4, 0.0, 256, 0.01, 1, (1,)),
    3: Workload(3, "llama2_7b_layer_kb3_ks1_s2pct_g8",
                (Shape("qkv", 4096, 12288), Shape("o", 4096, 4096), Shape("gate_up", 4096, 22016),
                 Shape("down", 11008, 4096)), 3, 1, 8, 0.02, None, 0.0, 32, (1,)),
    4: Workload(4, "llama2_7b_mlp_batch_kb2_ks1_s2pct_g4",
                (Shape("up_4096x11008", 4096, 11008), Shape("down_11008x4096", 11008, 4096)),
                2, 1, 4, 0.02, None, 0.0, 1, (1, 4, 8, 16)),
    5: Workload(5, "llama2_70b_layer_kb2_ks1_s3pct_g4",
                (Shape("qkv", 8192, 10240), Shape("o", 8192, 8192), Shape("gate_up", 8192, 57344),
                 Shape("down", 28672, 8192)), 2, 1, 4, 0.03, None, 0.0, 80, (1,)),
}


def workload_layer(cid: int, shape_idx: int = 0, layer: int = 0) -> Layer:
    wl = WORKLOADS[cid]
    sh = wl.shapes[shape_idx]
    return make_layer(sh.n, sh.k, wl.kb, wl.ks, wl.g, sal_frac=wl.sal_frac, s=wl.sal_fixed if wl.ks else None,
                      outlier_frac=wl.outlier_frac, seed=(cid, layer, shape_idx))


def workload_x(cid: int, layer_obj: Layer, batch: int, shape_idx: int = 0, layer: int = 0) -> np.ndarray:
    return make_x(layer_obj, batch, seed=(cid, layer, shape_idx))


# --------------------------------------------------------------------------
# Inputs of the offline decomposition (dense synthetic weights)
# --------------------------------------------------------------------------
# A synthetic stand-in for one trained linear layer: fp16 N(0, 0.02) entries
# scaled by a log-normal factor per row and per column (sigma 0.3), so that
# rows and columns differ in magnitude, the anisotropy the row-column
# decomposition is meant to capture.  Column weights of the weighted least
# squares stand in for the diagonal of the calibration Hessian 2 X X^T: the
# mean square of NCAL calibration draws of each input channel (same
# activation distribution and outlier channels as make_x).

T_W, T_W_ROW, T_W_COL = 20, 21, 22


def decomp_matrix(n: int, k: int, seed: tuple = (0, 0, 0)) -> np.ndarray:
    """fp16 [n][k] synthetic weights as raw uint16 bits."""
    v = stream(*seed, T_W).normal(0.0, 0.02, size=(n, k))
    v *= np.exp(stream(*seed, T_W_ROW).normal(0.0, 0.3, size=(n, 1)))
    v *= np.exp(stream(*seed, T_W_COL).normal(0.0, 0.3, size=(1, k)))
    return v.astype(np.float16).view(np.uint16)


def calibration_weights(k: int, outlier_frac: float = 0.0, seed: tuple = (0, 0, 0)) -> np.ndarray:
    """fp64 [k] per-column weights: mean over NCAL draws of fp16(x_j)^2."""
    outl = outlier_channels(stream(*seed, T_OUTLIER), k, outlier_frac)
    cal = stream(*seed, T_CAL).normal(0.0, 1.0, size=(NCAL, k))
    if outl.size:
        cal[:, outl] *= 20.0
    cal = cal.astype(np.float16).astype(np.float64)
    return (cal * cal).mean(axis=0)


# --------------------------------------------------------------------------
# Small structured inputs used by the exact-arithmetic tests
# --------------------------------------------------------------------------

def dyadic_layer(n: int, k: int, kb: int, ks: int, g: int, s: int, seed: int = 7) -> tuple:
    """A layer and activations whose every partial sum is exact in fp32.

    x in {-2..2} * 2^-3 (dyadic_x), c in {2^-2, 2^-1, 1}, r in {2^-1, 1}.  Returns the Layer.
    """
    rng = stream(99, seed)
    c_choices = np.array([0.25, 0.5, 1.0])
    r_choices = np.array([0.5, 1.0])

    def pick(choices, shape):
        return choices[rng.integers(0, len(choices), size=shape)].astype(np.float16).view(np.uint16)

    bits_g = np.stack([sign_words(rng, n, k) for _ in range(kb)]) if kb else np.zeros((0, n, words_per_row(k)), np.uint32)
    r_g = pick(r_choices, (kb, n))
    c_g = pick(c_choices, (kb, k))
    if ks and s:
        sal = np.sort(rng.choice(k, size=s, replace=False)).astype(np.int32)
        bits_s = np.stack([sign_words(rng, n, s) for _ in range(ks)])
        r_s = pick(r_choices, (ks, n))
        c_s = pick(c_choices, (ks, s))
    else:
        ks, s = 0, 0
        sal = np.zeros(0, np.int32)
        bits_s = np.zeros((0, n, 0), np.uint32)
        r_s = np.zeros((0, n), np.uint16)
        c_s = np.zeros((0, 0), np.uint16)
    layer = Layer(n, k, s, kb, ks, g, bits_g, r_g, c_g, bits_s, r_s, c_s, sal)
    return layer


def dyadic_grouped_layer(n: int, k: int, kb: int, ks: int, g: int, row_group: int, sal_group: int,
                         seed: int = 7) -> Layer:
    """Block-wise row-scale layer with the dyadic value sets of dyadic_layer (exact in fp32).

    Salient columns: sal_group random columns of every row_group-column block.
    """
    rng = stream(97, seed)
    c_choices = np.array([0.25, 0.5, 1.0])
    r_choices = np.array([0.5, 1.0])
    ng = (k + row_group - 1) // row_group

    def pick(choices, shape):
        return choices[rng.integers(0, len(choices), size=shape)].astype(np.float16).view(np.uint16)

    bits_g = np.stack([sign_words(rng, n, k) for _ in range(kb)])
    r_g = pick(r_choices, (kb, n, ng))
    c_g = pick(c_choices, (kb, k))
    if ks:
        sal = np.concatenate([np.sort(rng.choice(np.arange(g0, min(g0 + row_group, k)), size=sal_group,
                                                 replace=False)) for g0 in range(0, k, row_group)]).astype(np.int32)
        s = int(sal.size)
        bits_s = np.stack([sign_words(rng, n, s) for _ in range(ks)])
        r_s = pick(r_choices, (ks, n, ng))
        c_s = pick(c_choices, (ks, s))
    else:
        s, sal_group = 0, 0
        sal = np.zeros(0, np.int32)
        bits_s = np.zeros((0, n, 0), np.uint32)
        r_s = np.zeros((0, n, ng), np.uint16)
        c_s = np.zeros((0, 0), np.uint16)
    return Layer(n, k, s, kb, ks, g, bits_g, r_g, c_g, bits_s, r_s, c_s, sal, np.zeros(0, np.int64),
                 row_group, sal_group)


def dyadic_x(k: int, batch: int, seed: int = 8) -> np.ndarray:
    rng = stream(98, seed)
    v = rng.integers(-2, 3, size=(batch, k)) * 0.125
    return v.astype(np.float16).view(np.uint16)
