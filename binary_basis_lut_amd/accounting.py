"""Byte and operation accounting for one LUT GEMV call (host-side arithmetic only).

Algorithmic bytes are what the method must move per call on the weight side:
the packed sign words of every segment, the fp16 row and column scales and
the int32 salient index.  Activations and outputs are counted separately.
The dense fp16 work that the method avoids is not counted.

The operation counts follow the cost model of the FluxBin summary (appendix
C.1): a table-building term and a table-reading term for the K_b global
bases over the full input width and the K_s salient bases over |S| columns.
"""
from __future__ import annotations

import math


def segment_lengths(k: int, s: int, kb: int, ks: int):
    return [k] * kb + [s] * ks


def packed_sign_bytes(n: int, k: int, s: int, kb: int, ks: int) -> int:
    """Canonical packed sign words: ceil(L/32) uint32 per row per segment."""
    return sum(4 * n * ((L + 31) // 32) for L in segment_lengths(k, s, kb, ks))


def weight_bytes(n: int, k: int, s: int, kb: int, ks: int) -> int:
    """Per-call algorithmic weight-side bytes: sign words + fp16 r, c + int32 index."""
    scales = 2 * (kb + ks) * n + 2 * (kb * k + ks * s)
    index = 4 * s if ks else 0
    return packed_sign_bytes(n, k, s, kb, ks) + scales + index


def grouped_weight_bytes(n: int, k: int, kb: int, ks: int, row_group: int, sal_group: int) -> int:
    """Per-call weight-side bytes of the block-wise row-scale format.

    Sign words of every segment, one fp16 row scale per (row, group of
    `row_group` columns) per basis (global and salient alike), fp16 column
    scales, int32 index; the salient width is sal_group per group.
    """
    ng = -(-k // row_group)
    s = ng * sal_group if ks else 0
    row_scales = 2 * (kb + ks) * n * ng
    col_scales = 2 * (kb * k + ks * s)
    index = 4 * s if ks else 0
    return packed_sign_bytes(n, k, s, kb, ks) + row_scales + col_scales + index


def activation_bytes(n: int, k: int, batch: int) -> int:
    """fp16 x in and fp16 y out."""
    return 2 * batch * (k + n)


def lookups(n: int, k: int, s: int, kb: int, ks: int, g: int, batch: int) -> int:
    """Table reads (and fp32 accumulations) per call."""
    return batch * n * sum(math.ceil(L / g) for L in segment_lengths(k, s, kb, ks))


def table_entries(k: int, s: int, kb: int, ks: int, g: int, batch: int) -> int:
    """Distinct table entries per call (2^g per g-column sub-vector per segment per batch row)."""
    return batch * (1 << g) * sum(math.ceil(L / g) for L in segment_lengths(k, s, kb, ks))


def dense_f16_bytes(n: int, k: int, batch: int = 1) -> int:
    """Bytes a dense fp16 GEMV of the same shape reads and writes."""
    return 2 * n * k + activation_bytes(n, k, batch)


# ---------------------------------------------------------------------------
# The pages' own storage and shared-memory models (used to pin the reading of
# the printed numbers).
# ---------------------------------------------------------------------------

def pages_abw_bits(kb: int, ks: int, group: int, salient_per_group: int) -> float:
    """Average bits per weight of the pages' g128-style format (FluxBin summary, appendix C.2).

    Global part: one sign bit per weight and one fp16 row scale per (row, group)
    per basis.  Salient part: sign bits on `salient_per_group` of every `group`
    columns and one fp16 row scale per (row, group) per salient basis.  Column
    scales and the index are amortised over the rows and counted as zero.
    """
    glob = kb * (1.0 + 16.0 / group)
    sal = ks * (salient_per_group / group + 16.0 / group)
    return glob + sal


def pages_shared_memory_bytes(mu: int, batch: int, kb: int, mtile: int, ktile: int) -> int:
    """Shared memory of the pages' A100 kernel tile (FluxBin summary, appendix E.2).

    Batch-specific fp32 tables of 2^mu entries for every mu-column group of the
    k-tile and every basis, plus an fp32 accumulator per row, basis and batch row.
    """
    tables = batch * kb * (ktile // mu) * (1 << mu) * 4
    acc = batch * kb * mtile * 4
    return tables + acc
